// Split-N encode on bf16 matrix cores: for one (b, h), one split of the N
// tokens and up to 256 latents, compute the partial softmax statistics of
//     O_m = sum_n softmax_n(s <Q_m, K_n>) V_n
// i.e. a running max mu_m (log2 units), a sum lambda_m and an unnormalised
// accumulator acc_m[D].  It serves both encode calls of the route: the seed
// encode (Q = the latent seeds; FLARE++ abstract, the extra encode call) and
// FLARE's encode (Q = the synthesised queries; FLARE summary, "Основной
// механизм FLARE", encode step).  Splits are combined exactly by the merge
// kernel from these statistics, as the pages' token-sharded implementation
// combines per-device latent outputs with their softmax statistics (French
// technical summary, "Contributions Clés", multi-GPU context parallelism).
//
// Work decomposition.  A 256-thread workgroup owns one (b, h, split, latent
// group); its four waves own MBW 16-latent blocks each and share tiles of TN
// tokens of K and V.  Tiles travel HBM -> LDS by direct-to-LDS loads (no
// staging registers) through a ring of four slots: while tile t is consumed,
// the loads of tiles t+1 and t+2 are in flight and tile t+3's are issued.
// The slots are distinct LDS variables and the tile loop is unrolled by four,
// so each access names its slot statically and waiting for tile t's loads
// (s_waitcnt vmcnt) leaves the younger tiles' loads running.  16-byte chunks
// of each token row are XOR-swizzled in LDS (the fetching lane picks the
// chunk that belongs to its slot) so the matrix-core operand reads are free
// of bank conflicts.  Per 32-token step a wave computes S^T = K Q^T tiles
// (rows = tokens, cols = latents), turns them into softmax weights in
// registers, and accumulates O^T += V^T P^T; V's operand comes from the
// token-major tile through transposing LDS reads (ds_read_b64_tr_b16).
//
// Softmax arithmetic.  The query operand arrives pre-multiplied by
// c = s * log2(e) as a bf16 hi/lo pair (two MFMAs per tile, ~16 mantissa
// bits), and -mu_m enters as the MFMA accumulator input, so the tile is
// already t = c <Q_m, K_n> - mu_m and a weight is one exp2.  mu_m is either
//   * a bound: c ||Q_m|| max_n ||K_n|| (Cauchy-Schwarz), supplied by the
//     caller when it is known and keeps every exponent within [-100, 0]; no
//     per-score max is taken; or
//   * online: initialised from the first step's exact column max and raised
//     only when some value in a step exceeds mu_m + TAU (exp2(TAU) keeps
//     every weight and sum finite), at which point acc and lambda are
//     rescaled.  Both give the same softmax up to rounding (softmax is
//     invariant to a common shift).
// lambda_m sums the same bf16-rounded weights that enter the PV product.
#pragma once

#include "common.h"

namespace flarepp {

struct EncodeArgs {
  const __bf16* q_hi;  // pre-scaled query operand rows, padded to Mp (zero rows beyond M)
  const __bf16* q_lo;  // low part of the same
  int64_t q_sb, q_sh;  // element strides of the operand between batches / heads
  int64_t q_off;       // the operand rows of (b, h) start at b*q_sb + h*q_sh - q_off
  const __bf16* K;     // B x H x N x D
  const __bf16* V;     // B x H x N x D
  float* part;         // [G][Mp][J][D + 4] partial records (G = heads of this launch)
  float* knorm;        // [G][J] max squared key norm of each split, or null
  const float* bias;   // [G][Mp] mu_m bound (log2 units; +inf = use online), or null
  int H, N, Mp, J, chunk;
  int64_t bh0;         // first (b, h) of this launch: grid.y = lbh indexes (b, h) = bh0 + lbh
};

template <int D>
struct KOperand;
template <>
struct KOperand<32> {
  typedef bf16x8 T;
  static constexpr int kLen = 8;
  __device__ __forceinline__ static f32x4 mma(T a, T b, f32x4 c) { return mfma_k32(a, b, c); }
};
template <>
struct KOperand<16> {
  typedef bf16x4 T;
  static constexpr int kLen = 4;
  __device__ __forceinline__ static f32x4 mma(T a, T b, f32x4 c) { return mfma_k16(a, b, c); }
};

// ---- the LDS ring: four K slots and four V slots of one tile each
// (TN * D = 4096 bf16 = 8 KB for D = 16 and D = 32).
constexpr int kTileElems = 4096;
__shared__ __attribute__((aligned(16))) __bf16 enc_k0[kTileElems];
__shared__ __attribute__((aligned(16))) __bf16 enc_k1[kTileElems];
__shared__ __attribute__((aligned(16))) __bf16 enc_k2[kTileElems];
__shared__ __attribute__((aligned(16))) __bf16 enc_k3[kTileElems];
__shared__ __attribute__((aligned(16))) __bf16 enc_v0[kTileElems];
__shared__ __attribute__((aligned(16))) __bf16 enc_v1[kTileElems];
__shared__ __attribute__((aligned(16))) __bf16 enc_v2[kTileElems];
__shared__ __attribute__((aligned(16))) __bf16 enc_v3[kTileElems];
template <int I>
__device__ __forceinline__ __bf16* ring_k() {
  return I == 0 ? enc_k0 : I == 1 ? enc_k1 : I == 2 ? enc_k2 : enc_k3;
}
template <int I>
__device__ __forceinline__ __bf16* ring_v() {
  return I == 0 ? enc_v0 : I == 1 ? enc_v1 : I == 2 ? enc_v2 : enc_v3;
}

// Swizzle of the 16-byte chunks of token row t (D/8 chunks per row): the
// chunk holding elements 8u..8u+7 sits at position u ^ swz(t).
template <int D>
__device__ __forceinline__ int chunk_swz(int t) {
  return D == 32 ? ((t >> 2) & 3) : ((t >> 3) & 1);
}
// Element offset of (token t, element e) inside a tile slot.
template <int D>
__device__ __forceinline__ int slot_off(int t, int e) {
  return t * D + ((((e >> 3) ^ chunk_swz<D>(t)) << 3) | (e & 7));
}

#define FLAREPP_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define FLAREPP_GLB(p) ((__attribute__((address_space(1))) void*)(p))
// s_waitcnt with vmcnt <= n (n < 64); lgkmcnt and expcnt are not waited on.
#define FLAREPP_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | (((n) >> 4) << 14))

// Issue the direct-to-LDS loads of one tile into slot I: each wave fetches
// 2 KB of K and 2 KB of V (two 1 KB instructions each); lane l of an
// instruction fills LDS chunk base + 16 l and therefore fetches the (token,
// chunk) that the swizzle places there.  Tokens past the split re-read the
// split's last row (they receive zero weight), so every tile issues the same
// number of loads and the wait counts stay uniform.
template <int D, int I>
__device__ __forceinline__ void tile_dma(const __bf16* Kp, const __bf16* Vp, int tb, int n1, int wave, int lane) {
  constexpr int U = D / 8;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = wave * 2 + i;
    const int s = blk * 64 + lane;
    const int t = s / U;
    const int u = (s % U) ^ chunk_swz<D>(t);
    const int64_t src = (int64_t)min(tb + t, n1 - 1) * D + 8 * u;
    __builtin_amdgcn_global_load_lds(FLAREPP_GLB(Kp + src), FLAREPP_LDS(ring_k<I>() + blk * 512), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(FLAREPP_GLB(Vp + src), FLAREPP_LDS(ring_v<I>() + blk * 512), 16, 0, 0);
  }
}
constexpr int kDmaPerTile = 4;  // load instructions per wave per tile

// Per-wave register state of the encode: query operands, the shift entering
// each S^T tile as its accumulator input, the softmax statistics, and O^T.
template <int D, int MBW>
struct EncodeState {
  typedef typename KOperand<D>::T kop_t;
  kop_t qh[MBW], ql[MBW];
  f32x4 cb[MBW];
  float mu[MBW], lam[MBW];
  f32x4 acc[D / 16][MBW];
  bool first;
};

// One 32-token step of one wave: S^T tiles, softmax weights, O^T += V^T P^T.
// ONLINE: keep a running max (raised lazily); otherwise the shift is a bound.
// MASK (ragged last step only): tokens at or past n1 get weight zero.
template <int D, int MBW, bool ONLINE, bool MASK>
__device__ __forceinline__ void encode_step(EncodeState<D, MBW>& st, const __bf16* sK, const __bf16* sV,
                                            int ks, int sb, int n1, int g, int c16) {
  constexpr int KL = KOperand<D>::kLen;
  constexpr int DB = D / 16;
  constexpr float TAU = 8.0f;
  typedef typename KOperand<D>::T kop_t;
  const kop_t k0 = *reinterpret_cast<const kop_t*>(sK + slot_off<D>(ks * 32 + c16, KL * g));
  const kop_t k1 = *reinterpret_cast<const kop_t*>(sK + slot_off<D>(ks * 32 + 16 + c16, KL * g));
  f32x4 s0[MBW], s1[MBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
    s0[i] = KOperand<D>::mma(k0, st.qh[i], st.cb[i]);
    s1[i] = KOperand<D>::mma(k1, st.qh[i], st.cb[i]);
    s0[i] = KOperand<D>::mma(k0, st.ql[i], s0[i]);
    s1[i] = KOperand<D>::mma(k1, st.ql[i], s1[i]);
  }
  if (MASK) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool o0 = sb + 4 * g + r >= n1, o1 = sb + 16 + 4 * g + r >= n1;
#pragma unroll
      for (int i = 0; i < MBW; ++i) {
        if (o0) s0[i][r] = -INFINITY;
        if (o1) s1[i][r] = -INFINITY;
      }
    }
  }
  if (ONLINE) {
    float lm[MBW];
    bool hit = st.first;
#pragma unroll
    for (int i = 0; i < MBW; ++i) {
      lm[i] = fmaxf(max3(s0[i][0], s0[i][1], s0[i][2]),
                    max3(s0[i][3], s1[i][0], max3(s1[i][1], s1[i][2], s1[i][3])));
      hit |= lm[i] > TAU;
    }
    if (__builtin_expect(__any(hit), 0)) {
#pragma unroll
      for (int i = 0; i < MBW; ++i) {
        const float cm = max_over_rows(lm[i]);
        const float d = st.first ? cm : fmaxf(cm, 0.0f);
        st.mu[i] += d;
        const float al = fast_exp2(-d);
        st.lam[i] *= al;
#pragma unroll
        for (int db = 0; db < DB; ++db) st.acc[db][i] *= al;
        s0[i] -= d;
        s1[i] -= d;
        st.cb[i] = f32x4{-st.mu[i], -st.mu[i], -st.mu[i], -st.mu[i]};
      }
      st.first = false;
    }
  }
  bf16x8 p[MBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
    const bf16x2 p0 = pack_bf16(fast_exp2(s0[i][0]), fast_exp2(s0[i][1]));
    const bf16x2 p1 = pack_bf16(fast_exp2(s0[i][2]), fast_exp2(s0[i][3]));
    const bf16x2 p2 = pack_bf16(fast_exp2(s1[i][0]), fast_exp2(s1[i][1]));
    const bf16x2 p3 = pack_bf16(fast_exp2(s1[i][2]), fast_exp2(s1[i][3]));
    st.lam[i] = add_pair(p3, add_pair(p2, add_pair(p1, add_pair(p0, st.lam[i]))));
    p[i] = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
  // V^T operand: lane (row d = 16 db + c16, k-row g) needs V[tok][d] for the
  // eight tokens of its k-slots; one transposing read gives a lane four
  // tokens of its column when the 16 lanes of row g supply the 4-token x
  // 16-column block (lane r: token base + r/4, columns 16 db + 4 (r%4) ..+3).
  const int vt = ks * 32 + 4 * g + (c16 >> 2);
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int ve = 16 * db + 4 * (c16 & 3);
    const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sV + slot_off<D>(vt, ve)));
    const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sV + slot_off<D>(vt + 16, ve)));
    const bf16x8 vop = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
    for (int i = 0; i < MBW; ++i) st.acc[db][i] = mfma_k32(vop, p[i], st.acc[db][i]);
  }
}

// Largest squared key norm among the tile's tokens seen by this thread
// (every thread reads two 16-byte chunks; the chunks of one row sit in
// adjacent lanes).
template <int D>
__device__ __forceinline__ float tile_knorm(const __bf16* sK, int tid) {
  constexpr int U = D / 8;
  float best = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(sK + (tid + 256 * h) * 8);
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x2 pr = {x[2 * e], x[2 * e + 1]};
      ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
    }
    ss += __shfl_xor(ss, 1);
    if (U == 4) ss += __shfl_xor(ss, 2);
    best = fmaxf(best, ss);
  }
  return best;
}

// One tile of the ring (slot I holds tile t): wait for this wave's loads of
// tile t, barrier (every wave's part has landed, and every wave has finished
// tile t-1, whose slot is refilled next), issue tile t+3 into that slot, then
// consume tile t: whole 32-token steps, and a masked step if the split ends
// inside the tile.
template <int D, int MBW, bool KNORM, bool ONLINE, int I>
__device__ __forceinline__ void encode_tile(EncodeState<D, MBW>& st, const __bf16* Kp, const __bf16* Vp, int t,
                                            int n0, int n1, int tid, int wave, int lane, bool wave_active,
                                            int g, int c16, float& kn2) {
  constexpr int TN = kTileElems / D;
  FLAREPP_WAIT_VM(2 * kDmaPerTile);
  __builtin_amdgcn_s_barrier();
  tile_dma<D, (I + 3) & 3>(Kp, Vp, n0 + (t + 3) * TN, n1, wave, lane);
  if (KNORM) kn2 = fmaxf(kn2, tile_knorm<D>(ring_k<I>(), tid));
  if (!wave_active) return;
  const int tb = n0 + t * TN;
  const int full = min(TN / 32, (n1 - tb) / 32);
#pragma unroll 1
  for (int ks = 0; ks < full; ++ks)
    encode_step<D, MBW, ONLINE, false>(st, ring_k<I>(), ring_v<I>(), ks, tb + ks * 32, n1, g, c16);
  if (full < TN / 32 && tb + full * 32 < n1)
    encode_step<D, MBW, ONLINE, true>(st, ring_k<I>(), ring_v<I>(), full, tb + full * 32, n1, g, c16);
}

template <int D, int MBW, bool KNORM, bool ONLINE>
__device__ __forceinline__ void encode_tiles(EncodeState<D, MBW>& st, const __bf16* Kp, const __bf16* Vp, int n0,
                                             int n1, int tid, int wave, int lane, bool wave_active, int g, int c16,
                                             float& kn2) {
  constexpr int TN = kTileElems / D;
  const int ntiles = (n1 - n0 + TN - 1) / TN;
  tile_dma<D, 0>(Kp, Vp, n0, n1, wave, lane);
  tile_dma<D, 1>(Kp, Vp, n0 + TN, n1, wave, lane);
  tile_dma<D, 2>(Kp, Vp, n0 + 2 * TN, n1, wave, lane);
  for (int t = 0; t < ntiles; t += 4) {
    encode_tile<D, MBW, KNORM, ONLINE, 0>(st, Kp, Vp, t, n0, n1, tid, wave, lane, wave_active, g, c16, kn2);
    if (t + 1 >= ntiles) break;
    encode_tile<D, MBW, KNORM, ONLINE, 1>(st, Kp, Vp, t + 1, n0, n1, tid, wave, lane, wave_active, g, c16, kn2);
    if (t + 2 >= ntiles) break;
    encode_tile<D, MBW, KNORM, ONLINE, 2>(st, Kp, Vp, t + 2, n0, n1, tid, wave, lane, wave_active, g, c16, kn2);
    if (t + 3 >= ntiles) break;
    encode_tile<D, MBW, KNORM, ONLINE, 3>(st, Kp, Vp, t + 3, n0, n1, tid, wave, lane, wave_active, g, c16, kn2);
  }
  // the ring's trailing loads must land before the workgroup's LDS is released
  FLAREPP_WAIT_VM(0);
}

// BOUNDED: the shift may come from a.bias (the bound path, with the online
// path as fallback when a bound is unsafe); otherwise always online.
template <int D, int MBW, bool KNORM, bool BOUNDED>
__global__ __launch_bounds__(256, 2) void encode_split_bf16(EncodeArgs a) {
  constexpr int DB = D / 16;     // 16-row blocks of O^T
  constexpr int KL = KOperand<D>::kLen;
  typedef typename KOperand<D>::T kop_t;
  __shared__ float sRed[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int j = blockIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const int n0 = j * a.chunk;
  const int n1 = min(a.N, n0 + a.chunk);
  const int nMB = a.Mp >> 4;
  const int mb0 = (blockIdx.z * 4 + wave) * MBW;
  const bool wave_active = mb0 < nMB;

  const __bf16* Kp = a.K + bh * (int64_t)a.N * D;
  const __bf16* Vp = a.V + bh * (int64_t)a.N * D;

  // ---- query operands (B of S^T = K Q^T: lane holds column m, k = d) and shift
  EncodeState<D, MBW> st;
  bool need_online = !BOUNDED || a.bias == nullptr;
  {
    const int64_t qo = (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off;
#pragma unroll
    for (int i = 0; i < MBW; ++i) {
      const int mblk = mb0 + i;
      if (mblk < nMB) {
        const int m = mblk * 16 + c16;
        st.qh[i] = *reinterpret_cast<const kop_t*>(a.q_hi + qo + (int64_t)m * D + KL * g);
        st.ql[i] = *reinterpret_cast<const kop_t*>(a.q_lo + qo + (int64_t)m * D + KL * g);
        st.mu[i] = (BOUNDED && a.bias) ? a.bias[lbh * a.Mp + m] : 0.0f;
      } else {
        st.qh[i] = kop_t{};
        st.ql[i] = kop_t{};
        st.mu[i] = 0.0f;
      }
      need_online |= !(st.mu[i] <= 1e30f);
      st.lam[i] = 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db) st.acc[db][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const bool online = __any(need_online);
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
    if (online) st.mu[i] = 0.0f;
    st.cb[i] = f32x4{-st.mu[i], -st.mu[i], -st.mu[i], -st.mu[i]};
  }
  st.first = online;
  float kn2 = 0.0f;
  // the operand loads above must not be counted with the ring's loads
  FLAREPP_WAIT_VM(0);

  if (!BOUNDED || online)
    encode_tiles<D, MBW, KNORM, true>(st, Kp, Vp, n0, n1, tid, wave, lane, wave_active, g, c16, kn2);
  else
    encode_tiles<D, MBW, KNORM, false>(st, Kp, Vp, n0, n1, tid, wave, lane, wave_active, g, c16, kn2);

  // ---- partial records
  if (wave_active) {
    constexpr int PS = Part<D>::kStride;
#pragma unroll
    for (int i = 0; i < MBW; ++i) {
      const int mblk = mb0 + i;
      if (mblk >= nMB) break;
      const int m = mblk * 16 + c16;
      const float lt = sum_over_rows(st.lam[i]);
      float* rec = a.part + ((lbh * a.Mp + m) * (int64_t)a.J + j) * PS;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(rec + 16 * db + 4 * g) = st.acc[db][i];
      if (g == 0) {
        rec[D] = lt;
        rec[D + 1] = st.mu[i];
      }
    }
  }
  if (KNORM) {
    float x = kn2;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    if (lane == 0) sRed[wave] = x;
    __syncthreads();
    if (tid == 0 && blockIdx.z == 0)
      a.knorm[lbh * a.J + j] = fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3]));
  }
}

}  // namespace flarepp

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
// Work decomposition.  A workgroup of NW waves (4 or 8) owns one (b, h,
// split, latent group); each wave owns MBW 16-latent blocks and all share
// tiles of TN tokens of K and V.  Tiles travel HBM -> LDS by direct-to-LDS
// loads (no staging registers) through a ring of four slots, with the loads
// of the two tiles after the one being consumed in flight; the tile loop is
// unrolled by four so every slot address is static, and waiting for one
// tile's loads (s_waitcnt vmcnt) leaves the younger tile's loads running.
// 16-byte chunks
// of each token row are XOR-swizzled in LDS (the fetching lane picks the
// chunk that belongs to its slot) so the matrix-core operand reads are free
// of bank conflicts.  Per 32-token step a wave computes S^T = K Q^T tiles
// (rows = tokens, cols = latents), turns them into softmax weights in
// registers, and accumulates O^T += V^T P^T; V's operand comes from the
// token-major tile through transposing LDS reads (ds_read_b64_tr_b16).  The
// work of a step is software-pipelined over the wave's latent blocks so the
// matrix core and the VALU overlap (see EncodePipe).
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
// lambda_m sums the same bf16-rounded weights that enter the PV product
// (computed on the matrix core as a row of ones times P^T).
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

// ---- tile geometry and the LDS ring.  A slot holds one tile of K or V
// (TE bf16 = TN tokens x D); the ring has four K slots and four V slots in one
// kernel-local LDS array, the V slot of a tile right after its K slot, so
// that every operand read of a step is a lane base plus an offset that fits
// the instruction's 16-bit immediate.  Eight-wave workgroups (one per CU) use
// 16 KB slots (128 KB ring); four-wave workgroups use 8 KB slots so two fit
// per CU.
template <int D, int NW>
struct Ring {
  static constexpr int TE = NW == 8 ? 8192 : 4096;  // elements per slot
  static constexpr int TN = TE / D;                 // tokens per tile
  static constexpr int SPT = TN / 32;               // 32-token steps per tile
  static constexpr int DI = TE / 8 / 64 / NW;       // 1 KB loads per wave, operand and tile
  static constexpr int kDma = 2 * DI;               // loads per wave and tile
  template <int I>
  __device__ __forceinline__ static __bf16* k(__bf16* ring) {
    return ring + 2 * I * TE;
  }
  template <int I>
  __device__ __forceinline__ static __bf16* v(__bf16* ring) {
    return ring + (2 * I + 1) * TE;
  }
};

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

// s_waitcnt with vmcnt <= n (n < 64); lgkmcnt and expcnt are not waited on.
// The empty asm statements keep the compiler from moving memory accesses
// across the wait.
#define FLAREPP_WAIT_VM(n)                                                                      \
  do {                                                                                          \
    asm volatile("" ::: "memory");                                                              \
    __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | (((n) >> 4) << 14));    \
    asm volatile("" ::: "memory");                                                              \
  } while (0)

// Workgroup barrier without the memory wait that __syncthreads() implies
// (the ring's loads are waited for explicitly, per tile).
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One direct-to-LDS load: every lane fetches 16 bytes from its own global
// address into LDS at lds_base + 16 * lane.  Written as an asm statement (it
// has no register results) so that the compiler does not track the LDS
// write: its own bookkeeping would make every later LDS read of any ring
// slot wait for all loads in flight, which would serialise the ring.  The
// ring's waits are explicit (FLAREPP_WAIT_VM before each tile's barrier).
// M0 (the LDS base of the load) is set and consumed inside the statement; the
// compiler treats M0 as reserved and uses it nowhere else in this library
// (tests/test_kernel_asm.py checks the generated code for that).
__device__ __forceinline__ void dma16(const __bf16* src, const __bf16* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory");
}

// Issue the direct-to-LDS loads of one tile into slot I: the NW waves split
// the tile's 16-byte chunks of K and of V (instructions of 1 KB each); lane l
// of an instruction fills LDS chunk base + 16 l and therefore fetches the
// (token, chunk) that the swizzle places there.  Tokens past the split
// re-read the split's last row (they receive zero weight), so every tile
// issues the same number of loads and the wait counts stay uniform.
template <int D, int NW, int I>
__device__ __forceinline__ void tile_dma(__bf16* ring, const __bf16* Kp, const __bf16* Vp, int tb, int n1,
                                         int wave, int lane) {
  typedef Ring<D, NW> R;
  constexpr int U = D / 8;
#pragma unroll
  for (int i = 0; i < R::DI; ++i) {
    const int blk = wave * R::DI + i;
    const int s = blk * 64 + lane;
    const int t = s / U;
    const int u = (s % U) ^ chunk_swz<D>(t);
    const int64_t src = (int64_t)min(tb + t, n1 - 1) * D + 8 * u;
    dma16(Kp + src, R::template k<I>(ring) + blk * 512);
    dma16(Vp + src, R::template v<I>(ring) + blk * 512);
  }
}

// Per-wave register state of the encode: query operands, the shift entering
// each S^T tile as its accumulator input, the softmax statistics, and O^T.
// acc[DB] is the sum lambda: its tile is ONES^T P^T, whose row 0 carries the
// column sums of the bf16 weights (so lambda sums exactly the weights that
// enter O^T).
template <int D, int MBW>
struct EncodeState {
  typedef typename KOperand<D>::T kop_t;
  kop_t qh[MBW], ql[MBW];
  f32x4 cb[MBW];
  float mu[MBW];
  float qn2[MBW];  // ||c Q_m||^2 of the lane's latent (from the hi + lo operand)
  f32x4 acc[D / 16 + 1][MBW];
};

// Software pipeline over (step, latent block) pairs.  While block i's softmax
// runs on the VALU, the matrix core works on the S^T tiles of the next block
// and on the O^T update of the previous one; those are independent of block
// i, so the two units overlap within the wave.
template <int D>
struct EncodePipe {
  typedef typename KOperand<D>::T kop_t;
  kop_t k0, k1;           // K operands of the current step (two 16-token halves)
  f32x4 s0, s1;           // S^T tiles of the next (step, block)
  bf16x8 p;               // weights of the previous block, whose O^T update is pending
  bf16x8 v[D / 16];       // V^T operands of the previous block's step
};

// K operands (A of S^T = K Q^T: lane holds token row c16, k-chunk g) of step ks.
template <int D>
__device__ __forceinline__ void load_kop(const __bf16* sK, int ks, int g, int c16,
                                         typename KOperand<D>::T& k0, typename KOperand<D>::T& k1) {
  constexpr int KL = KOperand<D>::kLen;
  typedef typename KOperand<D>::T kop_t;
  k0 = *reinterpret_cast<const kop_t*>(sK + slot_off<D>(ks * 32 + c16, KL * g));
  k1 = *reinterpret_cast<const kop_t*>(sK + slot_off<D>(ks * 32 + 16 + c16, KL * g));
}

// V^T operands of step ks: lane (row d = 16 db + c16, k-row g) needs V[tok][d]
// for the eight tokens of its k-slots; one transposing read gives a lane four
// tokens of its column when the 16 lanes of row g supply the 4-token x
// 16-column block (lane r: token base + r/4, columns 16 db + 4 (r%4) ..+3).
template <int D>
__device__ __forceinline__ void load_vop(const __bf16* sV, int ks, int g, int c16, bf16x8 (&v)[D / 16]) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const int vt = ks * 32 + 4 * g + (c16 >> 2);
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    const int ve = 16 * db + 4 * (c16 & 3);
    const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sV + slot_off<D>(vt, ve)));
    const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sV + slot_off<D>(vt + 16, ve)));
    v[db] = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  }
}

// S^T tiles of latent block i (shift as accumulator input, query as hi + lo).
template <int D, int MBW>
__device__ __forceinline__ void block_logits(const EncodeState<D, MBW>& st, int i, typename KOperand<D>::T k0,
                                             typename KOperand<D>::T k1, f32x4& s0, f32x4& s1) {
  s0 = KOperand<D>::mma(k0, st.qh[i], st.cb[i]);
  s1 = KOperand<D>::mma(k1, st.qh[i], st.cb[i]);
  s0 = KOperand<D>::mma(k0, st.ql[i], s0);
  s1 = KOperand<D>::mma(k1, st.ql[i], s1);
}

__device__ __forceinline__ bf16x8 weights(f32x4 s0, f32x4 s1) {
  const bf16x2 p0 = pack_bf16(fast_exp2(s0[0]), fast_exp2(s0[1]));
  const bf16x2 p1 = pack_bf16(fast_exp2(s0[2]), fast_exp2(s0[3]));
  const bf16x2 p2 = pack_bf16(fast_exp2(s1[0]), fast_exp2(s1[1]));
  const bf16x2 p3 = pack_bf16(fast_exp2(s1[2]), fast_exp2(s1[3]));
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// O^T and lambda updates of block i from its weights p and its step's V^T operands.
template <int D, int MBW>
__device__ __forceinline__ void block_update(EncodeState<D, MBW>& st, int i, const bf16x8 (&v)[D / 16], bf16x8 p,
                                             bf16x8 ones) {
#pragma unroll
  for (int db = 0; db < D / 16; ++db) st.acc[db][i] = mfma_k32(v[db], p, st.acc[db][i]);
  st.acc[D / 16][i] = mfma_k32(ones, p, st.acc[D / 16][i]);
}

// One 32-token step (step ks of the V slot sV).  sKn / ksn locate the next
// step's K operands (HAS_NEXT).  Operand loads are placed right after the
// last use of the registers they replace: the next step's K after the last
// logits of this step's K, this step's V after the previous block's pending
// update; the pipeline registers are then overwritten in place instead of
// copied every step.  ONLINE: running max, starting from the exact column
// max of the split's first step and raised lazily (only when a value exceeds
// mu + TAU, so weights and sums stay finite); otherwise the shift is a bound.
// MASK (the split's ragged last step): tokens at or past n1 weigh zero.
template <int D, int MBW, bool ONLINE, bool MASK, bool HAS_NEXT>
__device__ __forceinline__ void encode_step(EncodeState<D, MBW>& st, EncodePipe<D>& pp, const __bf16* sV, int ks,
                                            const __bf16* sKn, int ksn, int sb, int n1, int g, int c16,
                                            bf16x8 ones) {
  constexpr int DB = D / 16;
  constexpr float TAU = 8.0f;
  if (HAS_NEXT && MBW == 1) load_kop<D>(sKn, ksn, g, c16, pp.k0, pp.k1);
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
    f32x4 s0 = pp.s0, s1 = pp.s1;
    // matrix core: next block's logits, previous block's update
    if (i + 1 < MBW) {
      block_logits<D, MBW>(st, i + 1, pp.k0, pp.k1, pp.s0, pp.s1);
      if (HAS_NEXT && i + 2 == MBW) load_kop<D>(sKn, ksn, g, c16, pp.k0, pp.k1);
    } else if (HAS_NEXT) {
      block_logits<D, MBW>(st, 0, pp.k0, pp.k1, pp.s0, pp.s1);
    }
    block_update<D, MBW>(st, i == 0 ? MBW - 1 : i - 1, pp.v, pp.p, ones);
    if (i == 0) load_vop<D>(sV, ks, g, c16, pp.v);
    // VALU: this block's weights
    if (MASK) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (sb + 4 * g + r >= n1) s0[r] = -INFINITY;
        if (sb + 16 + 4 * g + r >= n1) s1[r] = -INFINITY;
      }
    }
    bf16x8 p = weights(s0, s1);
    // keep the weights ahead of the (rare) rescale branch, in the same
    // scheduling region as the matrix-core work above
    asm volatile("" : "+v"(p));
    if (ONLINE) {
      const float lm = fmaxf(max3(s1[2], s1[3], max3(s0[3], s1[0], max3(s0[0], s0[1], s0[2]))), s1[1]);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(lm > TAU) != 0, 0)) {
        const float d = fmaxf(max_over_rows(lm), 0.0f);
        st.mu[i] += d;
        const float al = fast_exp2(-d);
#pragma unroll
        for (int db = 0; db <= DB; ++db) st.acc[db][i] *= al;
        s0 -= d;
        s1 -= d;
        if (MBW == 1) {  // the pending logits are this block's next step
          pp.s0 -= d;
          pp.s1 -= d;
        }
        st.cb[i] = f32x4{-st.mu[i], -st.mu[i], -st.mu[i], -st.mu[i]};
        p = weights(s0, s1);
      }
    }
    pp.p = p;
  }
}

// Largest squared key norm among the tokens of the K tile in slot I whose
// 16-byte chunks this lane loaded itself (the chunks of one token row are
// loaded by adjacent lanes), valid as soon as this wave's loads of the tile
// have landed.
template <int D, int NW, int I>
__device__ __forceinline__ float own_knorm(const __bf16* ring, int wave, int lane) {
  typedef Ring<D, NW> R;
  constexpr int U = D / 8;
  float best = 0.0f;
#pragma unroll
  for (int i = 0; i < R::DI; ++i) {
    const int blk = wave * R::DI + i;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(R::template k<I>(const_cast<__bf16*>(ring)) + blk * 512 + 8 * lane);
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

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt not waited on).
constexpr uint32_t kEncWaitLgkm0 = 0xF | (0x7 << 4) | (0x3 << 14);

// Ring protocol.  Tile u+2's loads are issued at the barrier that opens tile
// u; before it a wave waits for its own loads of tile u (those of tile u+1
// may still be in flight), so every wave's part of tile u has landed once all
// have arrived.  The barrier opening tile u is taken at the start of the last
// step of tile u-1, which still reads tile u-1 and (for the next step's K
// operands) tile u; the slot refilled there, (u+2) & 3, held tile u-2, which
// every wave has finished reading.
//
// TNORM: the barrier also publishes the largest squared key norm of tile u.
// Each wave reduces the norms of the chunks it loaded itself (landed after
// its wait) and stores the result in sKm[u & 1][wave] before the barrier;
// after it every wave takes the maximum over the NW entries.  Two buffers
// suffice: the entries of tile u are read right after the barrier that opens
// it, and rewritten (for tile u + 2) only after the next barrier.
template <int D, int NW, int I, bool TNORM>
__device__ __forceinline__ float ring_open(__bf16* ring, float* sKm, const __bf16* Kp, const __bf16* Vp, int u,
                                           int n0, int n1, int wave, int lane) {
  constexpr int kWait = Ring<D, NW>::kDma;
  FLAREPP_WAIT_VM(kWait);
  float* slot = sKm + (u & 1) * NW;
  if (TNORM) {
    const float part = wave_max(own_knorm<D, NW, I>(ring, wave, lane));
    if (lane == 0) slot[wave] = part;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kEncWaitLgkm0);  // the entry is in LDS before the barrier
  }
  ring_barrier();
  tile_dma<D, NW, (I + 2) & 3>(ring, Kp, Vp, n0 + (u + 2) * Ring<D, NW>::TN, n1, wave, lane);
  float km2 = 0.0f;
  if (TNORM) {
    km2 = slot[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) km2 = fmaxf(km2, slot[w]);
  }
  return km2;
}

// Tile t in slot I (already opened): its steps, the last of which opens tile
// t+1 (if any) and starts that tile's first logits.  CHECK: every step
// compares its scores with the running max (encode_step's online rule).
// With TNORM, km2 holds the largest squared key norm of tile t on entry and
// that of tile t+1 on exit.
template <int D, int NW, int MBW, bool TNORM, bool CHECK, int I>
__device__ __forceinline__ void encode_tile_steps(EncodeState<D, MBW>& st, EncodePipe<D>& pp, __bf16* ring,
                                                  float* sKm, const __bf16* Kp, const __bf16* Vp, int t, int n0,
                                                  int n1, int ntiles, int wave, int lane, bool wave_active, int g,
                                                  int c16, bf16x8 ones, float& km2) {
  typedef Ring<D, NW> R;
  constexpr int J1 = (I + 1) & 3;
  const int tb = n0 + t * R::TN;
  const int nsteps = min(R::SPT, (n1 - tb + 31) / 32);
#pragma unroll 1
  for (int ks = 0; ks + 1 < nsteps; ++ks) {
    if (wave_active)
      encode_step<D, MBW, CHECK, false, true>(st, pp, R::template v<I>(ring), ks, R::template k<I>(ring), ks + 1,
                                              tb + ks * 32, n1, g, c16, ones);
  }
  const int ks = nsteps - 1;
  if (t + 1 < ntiles) {
    km2 = ring_open<D, NW, J1, TNORM>(ring, sKm, Kp, Vp, t + 1, n0, n1, wave, lane);
    if (wave_active)
      encode_step<D, MBW, CHECK, false, true>(st, pp, R::template v<I>(ring), ks, R::template k<J1>(ring), 0,
                                              tb + ks * 32, n1, g, c16, ones);
  } else if (wave_active) {
    if (tb + (ks + 1) * 32 <= n1)
      encode_step<D, MBW, CHECK, false, false>(st, pp, R::template v<I>(ring), ks, nullptr, 0, tb + ks * 32, n1, g,
                                               c16, ones);
    else
      encode_step<D, MBW, CHECK, true, false>(st, pp, R::template v<I>(ring), ks, nullptr, 0, tb + ks * 32, n1, g,
                                              c16, ones);
  }
}

// Tile rule of the online path.  A score of latent m in a tile is at most
// ||c Q_m|| max_n ||K_n|| - mu_m (Cauchy-Schwarz, log2 units, maximum over
// the tile's tokens); when that bound is at most TAU_SKIP for every latent of
// the wave, no weight of the tile can exceed 2^TAU_SKIP (sums stay far from
// the float range), and the per-step comparison with the running max is
// skipped for the whole tile.  Otherwise (or for non-finite norms) every
// step checks.
template <int D, int MBW>
__device__ __forceinline__ bool tile_needs_check(const EncodeState<D, MBW>& st, float km2) {
  constexpr float TAU_SKIP = 32.0f;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
    // ||c Q_m|| sqrt(km2) <= mu_m + TAU_SKIP, squared (both sides >= 0)
    const float lim = st.mu[i] + TAU_SKIP;
    bad |= !(lim >= 0.0f && st.qn2[i] * km2 <= lim * lim);
  }
  return __builtin_amdgcn_ballot_w64(bad) != 0;
}

template <int D, int NW, int MBW, bool KNORM, bool ONLINE, bool SKIP, int I>
__device__ __forceinline__ void encode_tile(EncodeState<D, MBW>& st, EncodePipe<D>& pp, __bf16* ring, float* sKm,
                                            const __bf16* Kp, const __bf16* Vp, int t, int n0, int n1, int ntiles,
                                            int wave, int lane, bool wave_active, int g, int c16, bf16x8 ones,
                                            float& km2, float& kn2) {
  constexpr bool TNORM = KNORM || (ONLINE && SKIP);
  if (KNORM) kn2 = fmaxf(kn2, km2);
  if (ONLINE && (!SKIP || tile_needs_check<D, MBW>(st, km2)))
    encode_tile_steps<D, NW, MBW, TNORM, true, I>(st, pp, ring, sKm, Kp, Vp, t, n0, n1, ntiles, wave, lane,
                                                  wave_active, g, c16, ones, km2);
  else
    encode_tile_steps<D, NW, MBW, TNORM, false, I>(st, pp, ring, sKm, Kp, Vp, t, n0, n1, ntiles, wave, lane,
                                                   wave_active, g, c16, ones, km2);
}

// SKIP: the online path applies the tile rule (tile_needs_check); otherwise
// every step of the online path checks.
template <int D, int NW, int MBW, bool KNORM, bool ONLINE, bool SKIP>
__device__ __forceinline__ void encode_tiles(EncodeState<D, MBW>& st, __bf16* ring, float* sKm, const __bf16* Kp,
                                             const __bf16* Vp, int n0, int n1, int wave, int lane,
                                             bool wave_active, int g, int c16, float& kn2) {
  typedef Ring<D, NW> R;
  constexpr int DB = D / 16;
  constexpr bool TNORM = KNORM || (ONLINE && SKIP);
  const int ntiles = (n1 - n0 + R::TN - 1) / R::TN;
  // A operand of the lambda tile: row 0 all ones
  const __bf16 one = c16 == 0 ? (__bf16)1.0f : (__bf16)0.0f;
  const bf16x8 ones = {one, one, one, one, one, one, one, one};
  EncodePipe<D> pp;
  pp.p = bf16x8{};  // no update pending before the first block
#pragma unroll
  for (int db = 0; db < DB; ++db) pp.v[db] = bf16x8{};

  tile_dma<D, NW, 0>(ring, Kp, Vp, n0, n1, wave, lane);
  tile_dma<D, NW, 1>(ring, Kp, Vp, n0 + R::TN, n1, wave, lane);
  float km2 = ring_open<D, NW, 0, TNORM>(ring, sKm, Kp, Vp, 0, n0, n1, wave, lane);
  if (wave_active) {
    load_kop<D>(R::template k<0>(ring), 0, g, c16, pp.k0, pp.k1);
    if (ONLINE) {
      // the running max starts at the exact column max of the first step
      // (the shift is still zero here)
#pragma unroll
      for (int i = 0; i < MBW; ++i) {
        f32x4 s0, s1;
        block_logits<D, MBW>(st, i, pp.k0, pp.k1, s0, s1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (n0 + 4 * g + r >= n1) s0[r] = -INFINITY;
          if (n0 + 16 + 4 * g + r >= n1) s1[r] = -INFINITY;
        }
        const float lm = fmaxf(max3(s1[2], s1[3], max3(s0[3], s1[0], max3(s0[0], s0[1], s0[2]))), s1[1]);
        st.mu[i] = max_over_rows(lm);
        st.cb[i] = f32x4{-st.mu[i], -st.mu[i], -st.mu[i], -st.mu[i]};
      }
    }
    block_logits<D, MBW>(st, 0, pp.k0, pp.k1, pp.s0, pp.s1);
  }
  for (int t = 0; t < ntiles; t += 4) {
    encode_tile<D, NW, MBW, KNORM, ONLINE, SKIP, 0>(st, pp, ring, sKm, Kp, Vp, t, n0, n1, ntiles, wave, lane,
                                              wave_active, g, c16, ones, km2, kn2);
    if (t + 1 >= ntiles) break;
    encode_tile<D, NW, MBW, KNORM, ONLINE, SKIP, 1>(st, pp, ring, sKm, Kp, Vp, t + 1, n0, n1, ntiles, wave, lane,
                                              wave_active, g, c16, ones, km2, kn2);
    if (t + 2 >= ntiles) break;
    encode_tile<D, NW, MBW, KNORM, ONLINE, SKIP, 2>(st, pp, ring, sKm, Kp, Vp, t + 2, n0, n1, ntiles, wave, lane,
                                              wave_active, g, c16, ones, km2, kn2);
    if (t + 3 >= ntiles) break;
    encode_tile<D, NW, MBW, KNORM, ONLINE, SKIP, 3>(st, pp, ring, sKm, Kp, Vp, t + 3, n0, n1, ntiles, wave, lane,
                                              wave_active, g, c16, ones, km2, kn2);
  }
  // the last block's pending update
  if (wave_active) block_update<D, MBW>(st, MBW - 1, pp.v, pp.p, ones);
  // the ring's trailing loads must land before the workgroup's LDS is released
  FLAREPP_WAIT_VM(0);
}

// BOUNDED: the shift may come from a.bias (the bound path, with the online
// path as fallback when a bound is unsafe); otherwise always online.
template <int D, int NW, int MBW, bool KNORM, bool BOUNDED>
__global__ __launch_bounds__(64 * NW, 8 / NW) void encode_split_bf16(EncodeArgs a) {
  constexpr int DB = D / 16;     // 16-row blocks of O^T
  constexpr int KL = KOperand<D>::kLen;
  typedef typename KOperand<D>::T kop_t;
  __shared__ __attribute__((aligned(16))) __bf16 ring[8 * Ring<D, NW>::TE];
  __shared__ float sKm[2 * NW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4, c16 = lane & 15;
  const int j = blockIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const int n0 = j * a.chunk;
  const int n1 = min(a.N, n0 + a.chunk);
  const int nMB = a.Mp >> 4;
  const int mb0 = (blockIdx.z * NW + wave) * MBW;
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
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < KL; ++e) {
        const float x = (float)st.qh[i][e] + (float)st.ql[i][e];
        ss = fmaf(x, x, ss);
      }
      st.qn2[i] = sum_over_rows(ss);
#pragma unroll
      for (int db = 0; db <= DB; ++db) st.acc[db][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const bool online = __any(need_online);
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
    if (online) st.mu[i] = 0.0f;
    st.cb[i] = f32x4{-st.mu[i], -st.mu[i], -st.mu[i], -st.mu[i]};
  }
  float kn2 = 0.0f;
  // the operand loads above must not be counted with the ring's loads
  FLAREPP_WAIT_VM(0);

  if (!BOUNDED || online)
    encode_tiles<D, NW, MBW, KNORM, true, !BOUNDED>(st, ring, sKm, Kp, Vp, n0, n1, wave, lane, wave_active, g, c16, kn2);
  else
    encode_tiles<D, NW, MBW, KNORM, false, false>(st, ring, sKm, Kp, Vp, n0, n1, wave, lane, wave_active, g, c16, kn2);

  // ---- partial records
  if (wave_active) {
    constexpr int PS = Part<D>::kStride;
#pragma unroll
    for (int i = 0; i < MBW; ++i) {
      const int mblk = mb0 + i;
      if (mblk >= nMB) break;
      const int m = mblk * 16 + c16;
      float* rec = a.part + ((lbh * a.Mp + m) * (int64_t)a.J + j) * PS;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(rec + 16 * db + 4 * g) = st.acc[db][i];
      if (g == 0) {
        rec[D] = st.acc[DB][i][0];  // row 0 of the lambda tile
        rec[D + 1] = st.mu[i];
      }
    }
  }
  // kn2 is the maximum of the tile maxima, the same in every lane
  if (KNORM && tid == 0 && blockIdx.z == 0) a.knorm[lbh * a.J + j] = kn2;
}

}  // namespace flarepp

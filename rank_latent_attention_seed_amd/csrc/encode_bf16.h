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
// group); its four waves own MBW 16-latent blocks each and share K/V tiles of
// TN tokens staged through LDS (double buffered: global loads for tile t+1 are
// in flight while tile t is consumed).  Per 32-token step a wave computes
// S^T = K Q^T tiles (rows = tokens, cols = latents), turns them into softmax
// weights in registers, and accumulates O^T += V^T P^T on the matrix cores.
// V is written to LDS transposed ([d][token]) so that its A-operand slices
// are two 8-byte reads.
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
  float* part;         // [G][J][Mp][D + 4] partial records (G = heads of this launch)
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

template <int D, int MBW, bool KNORM>
__global__ __launch_bounds__(256, 2) void encode_split_bf16(EncodeArgs a) {
  constexpr int TN = 4096 / D;   // tokens per LDS tile: 8 KB of K
  constexpr int VROW = TN + 8;   // transposed-V row stride (elements); 4-dword skew per row
  constexpr int DB = D / 16;     // 16-row blocks of O^T
  constexpr int KL = KOperand<D>::kLen;
  constexpr int OCT = D / 8;     // 16-byte units per token row
  constexpr float TAU = 8.0f;
  typedef typename KOperand<D>::T kop_t;

  __shared__ __attribute__((aligned(16))) __bf16 sK[2][TN * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][D * VROW];
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

  // ---- query operands (B of S^T = K Q^T: lane holds column m, k = d) and bias
  kop_t qh[MBW], ql[MBW];
  f32x4 cb[MBW];
  float mu[MBW];
  bool online = true;
  {
    const int64_t qo = (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off;
    const __bf16* qhp = a.q_hi + qo;
    const __bf16* qlp = a.q_lo + qo;
    bool need_online = a.bias == nullptr;
#pragma unroll
    for (int i = 0; i < MBW; ++i) {
      const int mblk = mb0 + i;
      if (mblk < nMB) {
        const int m = mblk * 16 + c16;
        qh[i] = *reinterpret_cast<const kop_t*>(qhp + (int64_t)m * D + KL * g);
        ql[i] = *reinterpret_cast<const kop_t*>(qlp + (int64_t)m * D + KL * g);
        mu[i] = a.bias ? a.bias[lbh * a.Mp + m] : 0.0f;
      } else {
        qh[i] = kop_t{};
        ql[i] = kop_t{};
        mu[i] = 0.0f;
      }
      need_online |= !(mu[i] <= 1e30f);
    }
    online = __any(need_online);
#pragma unroll
    for (int i = 0; i < MBW; ++i) {
      if (online) mu[i] = 0.0f;
      cb[i] = f32x4{-mu[i], -mu[i], -mu[i], -mu[i]};
    }
  }
  bool first = online;

  f32x4 acc[DB][MBW];
  float lam[MBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
    lam[i] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float kn2 = 0.0f;

  // ---- staging of K/V tiles: K linear ([TN][D]), V transposed ([D][VROW])
  const int ntiles = (n1 - n0 + TN - 1) / TN;
  uint4 rk[2], rv[2];
  auto gload = [&](int t) {
    const int tb = n0 + t * TN;
#pragma unroll
    for (int u2 = 0; u2 < 2; ++u2) {
      const int u = tid + u2 * 256;
      const int tok = u / OCT, oc = u % OCT;
      rk[u2] = (tb + tok < n1)
                   ? *reinterpret_cast<const uint4*>(Kp + (int64_t)(tb + tok) * D + 8 * oc)
                   : make_uint4(0, 0, 0, 0);
    }
    const int p = tid / OCT, q = tid % OCT;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int tok = 2 * p + e;
      rv[e] = (tb + tok < n1)
                  ? *reinterpret_cast<const uint4*>(Vp + (int64_t)(tb + tok) * D + 8 * q)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int u2 = 0; u2 < 2; ++u2) {
      const int u = tid + u2 * 256;
      *reinterpret_cast<uint4*>(&sK[buf][u * 8]) = rk[u2];
      if (KNORM) {
        const bf16x8 x = __builtin_bit_cast(bf16x8, rk[u2]);
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 pr = {x[2 * e], x[2 * e + 1]};
          ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
        }
        ss += __shfl_xor(ss, 1);
        if (OCT == 4) ss += __shfl_xor(ss, 2);
        kn2 = fmaxf(kn2, ss);
      }
    }
    const int p = tid / OCT, q = tid % OCT;
    const uint32_t w0[4] = {rv[0].x, rv[0].y, rv[0].z, rv[0].w};
    const uint32_t w1[4] = {rv[1].x, rv[1].y, rv[1].z, rv[1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t lo = w0[e >> 1], hi = w1[e >> 1];
      const uint32_t pair = (e & 1) ? ((hi & 0xFFFF0000u) | (lo >> 16)) : ((hi << 16) | (lo & 0xFFFFu));
      *reinterpret_cast<uint32_t*>(&sV[buf][(8 * q + e) * VROW + 2 * p]) = pair;
    }
  };

  gload(0);
  swrite(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int tb = n0 + t * TN;
    if (wave_active) {
#pragma unroll 1
      for (int ks = 0; ks < TN / 32; ++ks) {
        const int sb = tb + ks * 32;
        if (sb >= n1) break;
        const kop_t k0 = *reinterpret_cast<const kop_t*>(&sK[buf][(ks * 32 + c16) * D + KL * g]);
        const kop_t k1 = *reinterpret_cast<const kop_t*>(&sK[buf][(ks * 32 + 16 + c16) * D + KL * g]);
        f32x4 s0[MBW], s1[MBW];
#pragma unroll
        for (int i = 0; i < MBW; ++i) {
          s0[i] = KOperand<D>::mma(k0, qh[i], cb[i]);
          s1[i] = KOperand<D>::mma(k1, qh[i], cb[i]);
          s0[i] = KOperand<D>::mma(k0, ql[i], s0[i]);
          s1[i] = KOperand<D>::mma(k1, ql[i], s1[i]);
        }
        if (sb + 32 > n1) {  // ragged tail: tokens past the split get no weight
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
        if (online) {
          float lm[MBW];
          bool hit = first;
#pragma unroll
          for (int i = 0; i < MBW; ++i) {
            lm[i] = fmaxf(max3(s0[i][0], s0[i][1], s0[i][2]),
                          max3(s0[i][3], s1[i][0], max3(s1[i][1], s1[i][2], s1[i][3])));
            hit |= lm[i] > TAU;
          }
          if (__any(hit)) {
#pragma unroll
            for (int i = 0; i < MBW; ++i) {
              const float cm = max_over_rows(lm[i]);
              const float d = first ? cm : fmaxf(cm, 0.0f);
              mu[i] += d;
              const float al = fast_exp2(-d);
              lam[i] *= al;
#pragma unroll
              for (int db = 0; db < DB; ++db) acc[db][i] *= al;
              s0[i] -= d;
              s1[i] -= d;
              cb[i] = f32x4{-mu[i], -mu[i], -mu[i], -mu[i]};
            }
            first = false;
          }
        }
        bf16x8 p[MBW];
#pragma unroll
        for (int i = 0; i < MBW; ++i) {
          const bf16x2 p0 = pack_bf16(fast_exp2(s0[i][0]), fast_exp2(s0[i][1]));
          const bf16x2 p1 = pack_bf16(fast_exp2(s0[i][2]), fast_exp2(s0[i][3]));
          const bf16x2 p2 = pack_bf16(fast_exp2(s1[i][0]), fast_exp2(s1[i][1]));
          const bf16x2 p3 = pack_bf16(fast_exp2(s1[i][2]), fast_exp2(s1[i][3]));
          lam[i] = add_pair(p3, add_pair(p2, add_pair(p1, add_pair(p0, lam[i]))));
          p[i] = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const __bf16* vrow = &sV[buf][(16 * db + c16) * VROW + ks * 32 + 4 * g];
          const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(vrow);
          const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(vrow + 16);
          const bf16x8 vop = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
          for (int i = 0; i < MBW; ++i) acc[db][i] = mfma_k32(vop, p[i], acc[db][i]);
        }
      }
    }
    if (t + 1 < ntiles) swrite((t + 1) & 1);
    __syncthreads();
  }

  // ---- partial records
  if (wave_active) {
    constexpr int PS = Part<D>::kStride;
#pragma unroll
    for (int i = 0; i < MBW; ++i) {
      const int mblk = mb0 + i;
      if (mblk >= nMB) break;
      const int m = mblk * 16 + c16;
      const float lt = sum_over_rows(lam[i]);
      float* rec = a.part + ((lbh * a.J + j) * (int64_t)a.Mp + m) * PS;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(rec + 16 * db + 4 * g) = acc[db][i];
      if (g == 0) {
        rec[D] = lt;
        rec[D + 1] = mu[i];
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

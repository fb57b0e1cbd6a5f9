// Spectrum of the routing's mixing matrix (FLARE summary, "Спектральный
// анализ": an eigendecomposition of the communication matrices in
// O(M^3 + M^2 N)).  The N x N mixing matrix W = W_dec W_enc (section
// "Матрица коммуникации низкого ранга") has the same nonzero eigenvalues as
// the M x M product C = W_enc W_dec.  Both factors are softmaxes of the same
// logits t_mn = c <Qd_m, K_n> (log2 units): W_enc[m, n] = 2^(t_mn - A_m)
// (encode, normalised over tokens; A_m is the encode's log-sum-exp) and
// W_dec[n, m] = 2^(t_mn - B_n) (decode, normalised over latents).  Hence
//     C = D_A^-1 E D_B^-1 E^T   with E_mn = 2^t_mn,
// which is similar (by D_A^1/2) to the symmetric positive semidefinite
//     G = F F^T,   F_mn = 2^(t_mn - (A_m + B_n) / 2),
// so the spectrum is real, in [0, 1] (C is row-stochastic), and equals the
// eigenvalues of G.  The kernels form G in O(M^2 N), split over tokens (for
// bf16 inputs on the matrix cores, with B_n formed in the same pass; for
// float32 inputs in float32 on the VALU), and find its eigenvalues in
// O(M^3): Householder reduction to tridiagonal form in LDS, then bisection
// with Sturm counts.
#pragma once

#include <float.h>

#include "common.h"

namespace flarepp {

constexpr int kSpecMaxM = 256;

template <typename KT>
__device__ __forceinline__ float load_elem(const KT* p, int64_t i) {
  return (float)p[i];
}

// Decode log-sum-exp of every token: B_n = log2 sum_m 2^t_mn.  One thread
// per token, Qd rows in LDS; the shift is the bound c ||k_n|| max ||Qd_m||
// when it keeps every exponent within [-100, 0], else an exact max.
struct SpecTokArgs {
  const float* q;  // Qd rows [G][M][D]
  const void* K;   // B x H x N x D
  float* tlse;     // [G][N]
  int H, N, M;
  int64_t bh0;
  float c;
};

template <int D, typename KT>
__global__ __launch_bounds__(256) void spectral_tokens(SpecTokArgs a) {
  __shared__ float sQ[kSpecMaxM * D];
  __shared__ float sQmax[4];
  const int tid = threadIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const float* qp = a.q + lbh * (int64_t)a.M * D;
  for (int e = tid; e < a.M * D; e += 256) sQ[e] = qp[e];
  __syncthreads();
  float qn2 = 0.0f;
  for (int m = tid; m < a.M; m += 256) {
    float n2 = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) n2 = fmaf(sQ[m * D + d], sQ[m * D + d], n2);
    qn2 = fmaxf(qn2, n2);
  }
  qn2 = wave_max(qn2);
  if ((tid & 63) == 0) sQmax[tid >> 6] = qn2;
  __syncthreads();
  const float qmax = sqrtf(fmaxf(fmaxf(sQmax[0], sQmax[1]), fmaxf(sQmax[2], sQmax[3])));
  const int n = blockIdx.x * 256 + tid;
  if (n >= a.N) return;
  const KT* kp = static_cast<const KT*>(a.K) + (bh * (int64_t)a.N + n) * D;
  float k[D], kn2 = 0.0f;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    k[d] = load_elem(kp, d);
    kn2 = fmaf(k[d], k[d], kn2);
  }
  auto logit = [&](int m) {
    float t = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) t = fmaf(k[d], sQ[m * D + d], t);
    return a.c * t;
  };
  float mu = fabsf(a.c) * sqrtf(kn2) * qmax * (1.0f + 1.0f / 4096.0f);  // bounds |logit| for either sign of c
  if (!(2.0f * mu <= 100.0f)) {
    mu = -INFINITY;
    for (int m = 0; m < a.M; ++m) mu = fmaxf(mu, logit(m));
  }
  float lam = 0.0f;
  for (int m = 0; m < a.M; ++m) lam += exp2f(logit(m) - mu);
  a.tlse[lbh * (int64_t)a.N + n] = mu + log2f(lam);
}

// Split partials of G = F F^T: workgroup (split j, head lbh) sums over its
// tokens, 32 at a time: the F tile (32 tokens x M latents) is formed in LDS,
// then thread (ti, tj) accumulates the 8 x 8 block G[8 ti .., 8 tj ..].
struct SpecGramArgs {
  const float* q;     // Qd rows [G][M][D]
  const void* K;
  const float* lse;   // encode log-sum-exp A_m, [G][Mp]
  const float* tlse;  // decode log-sum-exp B_n, [G][N]
  float* part;        // [G][J][M][M]
  int H, N, M, Mp, J, chunk;
  int64_t bh0;
  float c;
};

template <int D, typename KT>
__global__ __launch_bounds__(1024) void spectral_gram(SpecGramArgs a) {
  constexpr int TT = 32;
  __shared__ float sQ[kSpecMaxM * D];
  __shared__ __attribute__((aligned(16))) float sF[TT][kSpecMaxM];
  __shared__ float sK[TT * D];
  __shared__ float sAh[kSpecMaxM];
  __shared__ float sBh[TT];
  const int tid = threadIdx.x;
  const int j = blockIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int n0 = j * a.chunk, n1 = min(a.N, n0 + a.chunk);
  const float* qp = a.q + lbh * (int64_t)a.M * D;
  for (int e = tid; e < a.M * D; e += 1024) sQ[e] = qp[e];
  for (int m = tid; m < kSpecMaxM; m += 1024) sAh[m] = m < a.M ? 0.5f * a.lse[lbh * a.Mp + m] : 0.0f;
  const int ti = tid >> 5, tj = tid & 31;
  float acc[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[r][s] = 0.0f;
  const KT* kp = static_cast<const KT*>(a.K) + bh * (int64_t)a.N * D;
  for (int tb = n0; tb < n1; tb += TT) {
    const int cnt = min(TT, n1 - tb);
    __syncthreads();
    for (int e = tid; e < cnt * D; e += 1024) sK[e] = load_elem(kp, (int64_t)tb * D + e);
    for (int e = tid; e < cnt; e += 1024) sBh[e] = 0.5f * a.tlse[lbh * (int64_t)a.N + tb + e];
    __syncthreads();
    // F tile; latents past M and tokens past the split are zero
    for (int e = tid; e < TT * kSpecMaxM; e += 1024) {
      const int n = e / kSpecMaxM, m = e % kSpecMaxM;
      float f = 0.0f;
      if (n < cnt && m < a.M) {
        float t = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) t = fmaf(sQ[m * D + d], sK[n * D + d], t);
        f = exp2f(a.c * t - sAh[m] - sBh[n]);
      }
      sF[n][m] = f;
    }
    __syncthreads();
    for (int n = 0; n < cnt; ++n) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(&sF[n][8 * ti]);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(&sF[n][8 * ti + 4]);
      const f32x4 y0 = *reinterpret_cast<const f32x4*>(&sF[n][8 * tj]);
      const f32x4 y1 = *reinterpret_cast<const f32x4*>(&sF[n][8 * tj + 4]);
      const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      const float y[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int s = 0; s < 8; ++s) acc[r][s] = fmaf(x[r], y[s], acc[r][s]);
    }
  }
  float* out = a.part + (lbh * (int64_t)a.J + j) * a.M * a.M;
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int row = 8 * ti + r, col = 8 * tj + s;
      if (row < a.M && col < a.M) out[(int64_t)row * a.M + col] = acc[r][s];
    }
}

// G[lbh] = sum over splits (and a copy into the caller's B x H x M x M
// buffer when sym_out is set).
struct SpecReduceArgs {
  const float* part;  // [G][J][M][M]
  float* mat;         // [G][M][M]
  float* sym_out;     // [BH][M][M] or null
  int G, J, M;
  int64_t bh0;
};

__global__ __launch_bounds__(256) void spectral_reduce(SpecReduceArgs a) {
  const int64_t mm = (int64_t)a.M * a.M;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.G * mm) return;
  const int64_t lbh = idx / mm, e = idx % mm;
  float s = 0.0f;
  for (int j = 0; j < a.J; ++j) s += a.part[(lbh * a.J + j) * mm + e];
  a.mat[idx] = s;
  if (a.sym_out) a.sym_out[(a.bh0 + lbh) * mm + e] = s;
}

// ---- bf16 inputs: B_n and the Gram partials in one pass on the matrix cores.
//
// Workgroup (split j, head lbh), eight waves, 32 tokens per step.  Wave w
// forms the logits of latent blocks 2w, 2w + 1 (16 latents each) as
// S^T = K (c Qd)^T with the query as a bf16 hi/lo pair (the operands the
// encode used, so A_m and these logits agree); its C tiles leave each lane
// one latent and eight tokens, which is exactly a 16x16x32 MFMA operand over
// the step's 32 tokens (common.h).  The decode log-sum-exp of every token
// combines a (max, sum) pair per wave through LDS; then
// F_mn 2^15 = 2^(t_mn - A_m / 2 - B_n / 2 + 15) is rounded to fp16 (F <= 1,
// so the scaled value stays below fp16's largest finite 65504 and keeps
// fp16's full 11-bit precision down to F = 2^-29) and written to LDS as
// operand fragments.  The Gram product G += F F^T then runs as 16x16x32 fp16
// MFMAs over 16x16 tiles of the upper triangle, grouped into 4x4 super-blocks
// (four diagonal super-blocks of 10 tiles, six off-diagonal ones of 16) so
// that each wave reads 8 fragments per step for 16 or 20 MFMAs.  The result
// is scaled by 2^-30 when written; mirrored tiles complete the symmetric
// matrix.
struct SpecMfmaArgs {
  const __bf16* qhi;  // [G][Mp][D] bf16 hi of c * Qd (log2 units)
  const __bf16* qlo;  // [G][Mp][D] bf16 lo
  const __bf16* K;    // B x H x N x D
  const float* lse;   // encode log-sum-exp A_m, [G][Mp]
  float* part;        // [G][J][M][M]
  int N, M, Mp, J, chunk;
  int64_t bh0;
};

// Super-block jobs by number of 64-latent groups (ng = ceil(Mp / 64)) and
// wave: a first job (I, J), I == J for a diagonal super-block, and an
// optional second diagonal one; -1 for none.
__constant__ const int8_t kSpecJobI[4][8] = {
    {0, -1, -1, -1, -1, -1, -1, -1}, {0, 0, 1, -1, -1, -1, -1, -1}, {0, 0, 1, 0, 1, 2, -1, -1}, {0, 0, 0, 1, 1, 2, 0, 2}};
__constant__ const int8_t kSpecJobJ[4][8] = {
    {0, -1, -1, -1, -1, -1, -1, -1}, {1, 0, 1, -1, -1, -1, -1, -1}, {1, 2, 2, 0, 1, 2, -1, -1}, {1, 2, 3, 2, 3, 3, 0, 2}};
__constant__ const int8_t kSpecJob2[4][8] = {
    {-1, -1, -1, -1, -1, -1, -1, -1}, {-1, -1, -1, -1, -1, -1, -1, -1}, {-1, -1, -1, -1, -1, -1, -1, -1},
    {-1, -1, -1, -1, -1, -1, 1, 3}};

// max / sum over the 16 lanes of a row (lanes sharing l / 16); every lane of
// the row gets the result
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x124>(x));
  return fmaxf(x, dpp<0x128>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x124>(x);
  return x + dpp<0x128>(x);
}

template <int D>
__global__ __launch_bounds__(512) void spectral_gram_mfma(SpecMfmaArgs a) {
  static_assert(D == 16 || D == 32, "head dimension 16 or 32");
  constexpr int kBlocks = kSpecMaxM / 16;
  __shared__ __attribute__((aligned(16))) _Float16 sF[kBlocks * 64 * 8];  // [block][lane] fragments
  __shared__ __attribute__((aligned(16))) float sMu[8 * 32], sLam[8 * 32], sCn[8 * 32];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int j = blockIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int n0 = j * a.chunk, n1 = min(a.N, n0 + a.chunk);
  const int nb = a.Mp / 16, ng = (nb + 3) / 4;
  for (int e = tid; e < kBlocks * 64; e += 512) reinterpret_cast<f16x8*>(sF)[e] = f16x8{};

  // this wave's two latent blocks: query operands, validity, F exponent offset
  bf16x8 qh[2], ql[2];
  bool valid[2];
  float cm[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int blk = 2 * w + b, m = 16 * blk + l16;
    valid[b] = m < a.M;
    cm[b] = valid[b] ? 15.0f - 0.5f * a.lse[lbh * a.Mp + m] : -INFINITY;
    qh[b] = bf16x8{};
    ql[b] = bf16x8{};
    if (blk < nb) {
      const __bf16* hp = a.qhi + (lbh * a.Mp + m) * D;
      const __bf16* lp = a.qlo + (lbh * a.Mp + m) * D;
      if constexpr (D == 32) {
        qh[b] = *reinterpret_cast<const bf16x8*>(hp + 8 * g);
        ql[b] = *reinterpret_cast<const bf16x8*>(lp + 8 * g);
      } else {  // k slots 0..15 take the hi operand, 16..31 the lo one (K is repeated)
        qh[b] = *reinterpret_cast<const bf16x8*>((g < 2 ? hp : lp) + 8 * (g & 1));
      }
    }
  }
  // K rows of a step: lane reads token tb + 16 h + l16, elements 8 (g mod D/8) ..
  // (a resource from the step's first token, so offsets stay small; tokens
  // past N read as zeros)
  const __bf16* khead = a.K + bh * (int64_t)a.N * D;
  const int kcol = D == 32 ? 8 * g : 8 * (g & 1);
  auto load_k = [&](int tb, int h) {
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(khead + (int64_t)tb * D, (uint32_t)((int64_t)(a.N - tb) * D * 2));
    return buffer_load<bf16x8>(kr, ((16 * h + l16) * D + kcol) * 2);
  };

  const int jobI = kSpecJobI[ng - 1][w], jobJ = kSpecJobJ[ng - 1][w], job2 = kSpecJob2[ng - 1][w];
  f32x4 acc[20];
#pragma unroll
  for (int t = 0; t < 20; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  auto frag = [&](int blk) { return *reinterpret_cast<const f16x8*>(sF + (blk * 64 + lane) * 8); };

  bf16x8 kc0 = load_k(n0, 0), kc1 = load_k(n0, 1);
  __syncthreads();
  for (int tb = n0; tb < n1; tb += 32) {
    const bf16x8 k0 = kc0, k1 = kc1;
    if (tb + 32 < n1) {
      kc0 = load_k(tb + 32, 0);
      kc1 = load_k(tb + 32, 1);
    }
    // logits: T[b][h][r] = t(latent 16 (2w + b) + l16, token 16 h + 4 g + r)
    f32x4 T[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      T[b][0] = mfma_k32(k0, qh[b], z);
      T[b][1] = mfma_k32(k1, qh[b], z);
      if constexpr (D == 32) {
        T[b][0] = mfma_k32(k0, ql[b], T[b][0]);
        T[b][1] = mfma_k32(k1, ql[b], T[b][1]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) T[b][h][r] = valid[b] ? T[b][h][r] : -INFINITY;
    }
    // per-token (max, sum) over this wave's latents
    f32x4 mu[2], lam[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float m = row16_max(fmaxf(T[0][h][r], T[1][h][r]));
        const float sh = m == -INFINITY ? 0.0f : m;
        mu[h][r] = m;
        lam[h][r] = row16_sum(fast_exp2(T[0][h][r] - sh) + fast_exp2(T[1][h][r] - sh));
      }
    if (l16 == 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        *reinterpret_cast<f32x4*>(sMu + w * 32 + 16 * h + 4 * g) = mu[h];
        *reinterpret_cast<f32x4*>(sLam + w * 32 + 16 * h + 4 * g) = lam[h];
      }
    }
    __syncthreads();
    // B_n of token tb + (lane mod 32), then -B_n / 2 (or -inf past the split)
    {
      const int t = lane & 31;
      float m = -INFINITY;
#pragma unroll
      for (int v = 0; v < 8; ++v) m = fmaxf(m, sMu[v * 32 + t]);
      float sum = 0.0f;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float mv = sMu[v * 32 + t];
        sum += mv == -INFINITY ? 0.0f : sLam[v * 32 + t] * fast_exp2(mv - m);
      }
      const float cn = tb + t < n1 ? -0.5f * (m + log2f(sum)) : -INFINITY;
      if (lane < 32) sCn[w * 32 + t] = cn;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const f32x4 cn0 = *reinterpret_cast<const f32x4*>(sCn + w * 32 + 4 * g);
    const f32x4 cn1 = *reinterpret_cast<const f32x4*>(sCn + w * 32 + 16 + 4 * g);
    // F fragments of the wave's blocks
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (2 * w + b < nb) {
        const f16x2 p0 = pack_f16(fast_exp2(T[b][0][0] + cn0[0] + cm[b]), fast_exp2(T[b][0][1] + cn0[1] + cm[b]));
        const f16x2 p1 = pack_f16(fast_exp2(T[b][0][2] + cn0[2] + cm[b]), fast_exp2(T[b][0][3] + cn0[3] + cm[b]));
        const f16x2 p2 = pack_f16(fast_exp2(T[b][1][0] + cn1[0] + cm[b]), fast_exp2(T[b][1][1] + cn1[1] + cm[b]));
        const f16x2 p3 = pack_f16(fast_exp2(T[b][1][2] + cn1[2] + cm[b]), fast_exp2(T[b][1][3] + cn1[3] + cm[b]));
        *reinterpret_cast<f16x8*>(sF + ((2 * w + b) * 64 + lane) * 8) =
            f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      }
    }
    __syncthreads();
    // Gram tiles of this wave's super-blocks
    if (jobI >= 0) {
      if (jobI != jobJ) {
        f16x8 fa[4], fb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          fa[u] = frag(4 * jobI + u);
          fb[u] = frag(4 * jobJ + u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[4 * u + v] = mfma_k32(fa[u], fb[v], acc[4 * u + v]);
      } else {
        f16x8 fa[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) fa[u] = frag(4 * jobI + u);
        int t = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = u; v < 4; ++v, ++t) acc[t] = mfma_k32(fa[u], fa[v], acc[t]);
        if (job2 >= 0) {
#pragma unroll
          for (int u = 0; u < 4; ++u) fa[u] = frag(4 * job2 + u);
          t = 10;
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = u; v < 4; ++v, ++t) acc[t] = mfma_k32(fa[u], fa[v], acc[t]);
        }
      }
    }
  }
  // G partial: c[r] = G[16 bi + 4 g + r][16 bj + l16] (times 2^30)
  float* out = a.part + (lbh * a.J + j) * (int64_t)a.M * a.M;
  auto put = [&](int bi, int bj, f32x4 c) {
    const int col = 16 * bj + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * bi + 4 * g + r;
      if (row < a.M && col < a.M) {
        const float x = c[r] * 0x1p-30f;
        out[(int64_t)row * a.M + col] = x;
        if (bi != bj) out[(int64_t)col * a.M + row] = x;
      }
    }
  };
  if (jobI >= 0) {
    if (jobI != jobJ) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) put(4 * jobI + u, 4 * jobJ + v, acc[4 * u + v]);
    } else {
      int t = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = u; v < 4; ++v, ++t) put(4 * jobI + u, 4 * jobI + v, acc[t]);
      if (job2 >= 0) {
        t = 10;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = u; v < 4; ++v, ++t) put(4 * job2 + u, 4 * job2 + v, acc[t]);
      }
    }
  }
}

// Eigenvalues of the symmetric G[lbh] (its lower triangle), one workgroup per
// head.  The lower triangle is held packed in LDS (at most 256 * 257 / 2
// floats, 131.6 KB).  Householder reduction to tridiagonal form (Golub & Van
// Loan, "Householder tridiagonalization"): for k = 0 .. M - 3 the reflector
// H = I - beta v v^T with v = x - alpha e_1, alpha = -sign(x_1) ||x||, maps
// the column x = A[k+1:, k] to alpha e_1; the trailing block becomes
// H A' H = A' - v w^T - w v^T with p = beta A' v, w = p - (beta v^T p / 2) v.
// Then every eigenvalue of the tridiagonal (d, e) by bisection on its
// Gershgorin interval: the number of eigenvalues below x is the number of
// negative terms of the Sturm sequence q_0 = d_0 - x,
// q_i = d_i - x - e_{i-1}^2 / q_{i-1} (tiny pivots replaced by -pivmin, as in
// LAPACK's bisection; the division by the hardware reciprocal, 1 ulp, so the
// count is that of a tridiagonal within a few ulp of (d, e)), four threads per
// eigenvalue counting at four points that cut its interval into fifths,
// until the interval is below 2 ulp of the spectrum's scale.  Output by
// decreasing value, eig[(bh0 + lbh) * M ...].
struct EigArgs {
  const float* mat;  // [G][M][M]
  float* eig;        // [BH][M]
  int M;
  int64_t bh0;
};

__device__ __forceinline__ int tri_at(int i, int j) { return i * (i + 1) / 2 + j; }  // j <= i

__global__ __launch_bounds__(1024) void tridiag_eigvals(EigArgs a) {
  __shared__ float sA[kSpecMaxM * (kSpecMaxM + 1) / 2];
  __shared__ float sv[kSpecMaxM], sp[kSpecMaxM], sd[kSpecMaxM], se[kSpecMaxM], se2[kSpecMaxM];
  __shared__ float sred[16];
  __shared__ float sbeta;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = a.M;
  const float* A = a.mat + blockIdx.x * (int64_t)M * M;
  for (int e = tid; e < M * M; e += 1024) {
    const int i = e / M, j = e - i * M;
    if (j <= i) sA[tri_at(i, j)] = A[e];
  }
  __syncthreads();
  for (int k = 0; k + 2 < M; ++k) {
    const int n = M - 1 - k, r0 = k + 1;  // trailing block: rows and columns r0 .. M - 1
    if (wave == 0) {
      float x[4], s = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = lane + 64 * q;
        x[q] = i < n ? sA[tri_at(r0 + i, k)] : 0.0f;
        if (i >= 1) s = fmaf(x[q], x[q], s);
      }
      s = wave_sum(s);
      const float x0 = sA[tri_at(r0, k)];
      float alpha = x0, beta = 0.0f, v0 = 0.0f;
      if (s > 0.0f) {
        alpha = -copysignf(sqrtf(fmaf(x0, x0, s)), x0);
        v0 = x0 - alpha;
        beta = -1.0f / (alpha * v0);  // 2 / v^T v, since v^T v = -2 alpha v0
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = lane + 64 * q;
        if (i < n) sv[i] = i == 0 ? v0 : x[q];
      }
      if (lane == 0) {
        sbeta = beta;
        sd[k] = sA[tri_at(k, k)];
        se[k] = alpha;
      }
    }
    __syncthreads();
    const float beta = sbeta;
    if (beta != 0.0f) {
      // p = beta A' v: four threads per row (thread 4 i + q takes the columns
      // q, q + 4, ...), a two-step reduction within the quad; then each
      // wave's part of v^T p
      const int i = tid >> 2, q = tid & 3;
      float acc = 0.0f;
      if (i < n) {
        const int gi = r0 + i;
        // columns j <= i: row gi of the packed triangle, contiguous (four
        // independent sums so the LDS reads of four columns overlap)
        const float* row = sA + tri_at(gi, r0);
        float a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
        int jj = q;
        for (; jj + 12 <= i; jj += 16) {
          acc = fmaf(row[jj], sv[jj], acc);
          a1 = fmaf(row[jj + 4], sv[jj + 4], a1);
          a2 = fmaf(row[jj + 8], sv[jj + 8], a2);
          a3 = fmaf(row[jj + 12], sv[jj + 12], a3);
        }
        for (; jj <= i; jj += 4) acc = fmaf(row[jj], sv[jj], acc);
        // columns j > i: entry (r0 + j, gi); offsets advance by
        // tri(x + 4) - tri(x) = 4 x + 10 between the thread's columns
        if (jj < n) {
          int off = tri_at(r0 + jj, gi);
          for (; jj + 12 < n; jj += 16) {
            const int o1 = off + 4 * (r0 + jj) + 10;
            const int o2 = o1 + 4 * (r0 + jj + 4) + 10;
            const int o3 = o2 + 4 * (r0 + jj + 8) + 10;
            acc = fmaf(sA[off], sv[jj], acc);
            a1 = fmaf(sA[o1], sv[jj + 4], a1);
            a2 = fmaf(sA[o2], sv[jj + 8], a2);
            a3 = fmaf(sA[o3], sv[jj + 12], a3);
            off = o3 + 4 * (r0 + jj + 12) + 10;
          }
          for (; jj < n; jj += 4) {
            acc = fmaf(sA[off], sv[jj], acc);
            off += 4 * (r0 + jj) + 10;
          }
        }
        acc = (acc + a1) + (a2 + a3);
      }
      acc += dpp<0xB1>(acc);  // quad_perm [1,0,3,2]
      acc += dpp<0x4E>(acc);  // quad_perm [2,3,0,1]
      acc *= beta;
      float vp = 0.0f;
      if (i < n && q == 0) {
        sp[i] = acc;
        vp = acc * sv[i];
      }
      vp = wave_sum(vp);
      if (lane == 0) sred[wave] = vp;
    }
    __syncthreads();
    if (beta != 0.0f) {
      float vtp = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) vtp += sred[v];
      const float kc = 0.5f * beta * vtp;
      // w_j = p_j - kc v_j for this lane's columns (lane + 64 c), once per step
      float vl[4], wl[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int jj = lane + 64 * c;
        vl[c] = jj < n ? sv[jj] : 0.0f;
        wl[c] = jj < n ? sp[jj] - kc * vl[c] : 0.0f;
      }
      // rows i = wave, wave + 16, ...: A'_ij -= v_i w_j + w_i v_j for j <= i,
      // four rows per pass, every load of a pass issued before its stores
      for (int i0 = wave; i0 < n; i0 += 64) {
        float x[4][4], vr[4], wr[4];
        float* rows[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + 16 * u;
          const bool live = i < n;
          vr[u] = live ? sv[i] : 0.0f;
          wr[u] = live ? sp[i] - kc * vr[u] : 0.0f;
          rows[u] = sA + tri_at(r0 + (live ? i : i0), r0);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int jj = lane + 64 * c;
            x[u][c] = live && jj <= i ? rows[u][jj] : 0.0f;
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + 16 * u;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int jj = lane + 64 * c;
            if (i < n && jj <= i) rows[u][jj] = x[u][c] - fmaf(vr[u], wl[c], wr[u] * vl[c]);
          }
        }
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    if (M >= 2) {
      sd[M - 2] = sA[tri_at(M - 2, M - 2)];
      se[M - 2] = sA[tri_at(M - 1, M - 2)];
    }
    sd[M - 1] = sA[tri_at(M - 1, M - 1)];
  }
  __syncthreads();
  for (int i = tid; i < M; i += 1024) se2[i] = se[i] * se[i];
  __syncthreads();
  // multisection: the four threads of a quad share eigenvalue e = tid / 4 and
  // count at four interior points of its interval, which then shrinks five-fold
  const int e = tid >> 2, sub = tid & 3;
  if (e >= M) return;  // whole quads leave together
  float glo = INFINITY, ghi = -INFINITY, e2max = 0.0f;
  for (int i = 0; i < M; ++i) {
    const float r = (i > 0 ? fabsf(se[i - 1]) : 0.0f) + (i + 1 < M ? fabsf(se[i]) : 0.0f);
    glo = fminf(glo, sd[i] - r);
    ghi = fmaxf(ghi, sd[i] + r);
    if (i + 1 < M) e2max = fmaxf(e2max, se2[i]);
  }
  const float scale = fmaxf(fabsf(glo), fabsf(ghi));
  const float pivmin = FLT_MIN * fmaxf(1.0f, e2max);
  const float tol = 2.0f * FLT_EPSILON * scale + FLT_MIN;
  float lo = glo - tol, hi = ghi + tol;
  for (int it = 0; it < 64 && hi - lo > tol; ++it) {
    const float step = (hi - lo) * 0.2f;
    const float x = lo + step * (float)(sub + 1);
    int cnt = 0;
    float q = sd[0] - x;
    for (int i = 0;; ++i) {
      if (fabsf(q) < pivmin) q = -pivmin;
      cnt += q < 0.0f;
      if (i + 1 == M) break;
      q = (sd[i + 1] - x) - se2[i] * __builtin_amdgcn_rcpf(q);
    }
    const float c = (float)cnt;
    const float cs[4] = {dpp<0x00>(c), dpp<0x55>(c), dpp<0xAA>(c), dpp<0xFF>(c)};
    float nlo = lo + step * 4.0f, nhi = hi;  // no count above e: the last fifth
#pragma unroll
    for (int k = 3; k >= 0; --k)
      if (cs[k] > (float)e) {
        nhi = lo + step * (float)(k + 1);
        nlo = k == 0 ? lo : lo + step * (float)k;
      }
    lo = nlo;
    hi = nhi;
  }
  if (sub == 0) a.eig[(a.bh0 + blockIdx.x) * M + (M - 1 - e)] = 0.5f * (lo + hi);
}

}  // namespace flarepp

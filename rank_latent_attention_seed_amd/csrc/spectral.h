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
// eigenvalues of G.  The kernels form G in O(M^2 N) (split over tokens) and
// find its eigenvalues with a parallel cyclic Jacobi iteration in O(M^3).
// Float32 arithmetic throughout.
#pragma once

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

// Eigenvalues of the symmetric G[lbh] (overwritten) by cyclic Jacobi: in each
// round the M (rounded up to even) indices form disjoint pairs (round-robin
// tournament, a "bye" for the padding index); every pair's rotation
// J = [[c, s], [-s, c]] with t = tan(theta) from
// tau = (a_qq - a_pp) / (2 a_pq), t = sign(tau) / (|tau| + sqrt(1 + tau^2))
// zeroes a_pq (Golub & Van Loan, the symmetric Schur decomposition), and
// A <- J^T A J is applied to all pairs at once, rows first, then columns
// (disjoint rotations commute).  A sweep is M - 1 rounds (every pair once);
// sweeps repeat until the off-diagonal Frobenius norm is below tol times the
// whole norm, at most max_sweeps times.  Output: eigenvalues by decreasing
// value, eig[(bh0 + lbh) * M ...].
struct JacobiArgs {
  float* mat;  // [G][M][M]
  float* eig;  // [BH][M]
  int M, max_sweeps;
  int64_t bh0;
  float tol;
};

__global__ __launch_bounds__(256) void jacobi_eigvals(JacobiArgs a) {
  __shared__ float sc[kSpecMaxM / 2], ss[kSpecMaxM / 2];
  __shared__ int sp[kSpecMaxM / 2], sq[kSpecMaxM / 2];
  __shared__ float sred[2][4];
  __shared__ float sdiag[kSpecMaxM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = a.M;
  const int64_t lbh = blockIdx.x;
  float* A = a.mat + lbh * (int64_t)M * M;
  const int n = (M + 1) & ~1;
  const int npairs = n / 2;
  for (int sweep = 0; sweep < a.max_sweeps; ++sweep) {
    // convergence test on the current matrix
    float off = 0.0f, all = 0.0f;
    for (int e = tid; e < M * M; e += 256) {
      const float x = A[e];
      all += x * x;
      if (e / M != e % M) off += x * x;
    }
    off = wave_sum(off);
    all = wave_sum(all);
    if (lane == 0) {
      sred[0][wave] = off;
      sred[1][wave] = all;
    }
    __syncthreads();
    const float offt = sred[0][0] + sred[0][1] + sred[0][2] + sred[0][3];
    const float allt = sred[1][0] + sred[1][1] + sred[1][2] + sred[1][3];
    __syncthreads();
    if (!(offt > a.tol * a.tol * allt)) break;
    for (int r = 0; r < n - 1; ++r) {
      if (tid < npairs) {
        int p, q;
        if (tid == 0) {
          p = r;
          q = n - 1;
        } else {
          p = (r + tid) % (n - 1);
          q = (r - tid + n - 1) % (n - 1);
        }
        if (p > q) {
          const int t = p;
          p = q;
          q = t;
        }
        float c = 1.0f, s = 0.0f;
        if (q < M) {
          const float apq = A[(int64_t)p * M + q];
          if (apq != 0.0f) {
            const float tau = (A[(int64_t)q * M + q] - A[(int64_t)p * M + p]) / (2.0f * apq);
            const float t = (tau >= 0.0f ? 1.0f : -1.0f) / (fabsf(tau) + sqrtf(1.0f + tau * tau));
            c = 1.0f / sqrtf(1.0f + t * t);
            s = t * c;
          }
        }
        sp[tid] = p;
        sq[tid] = q;
        sc[tid] = c;
        ss[tid] = s;
      }
      __syncthreads();
      // rows p, q of every pair: A <- J^T A
      for (int e = tid; e < npairs * M; e += 256) {
        const int k = e / M, col = e % M;
        const int p = sp[k], q = sq[k];
        if (q >= M) continue;
        const float c = sc[k], s = ss[k];
        const float ap = A[(int64_t)p * M + col], aq = A[(int64_t)q * M + col];
        A[(int64_t)p * M + col] = c * ap - s * aq;
        A[(int64_t)q * M + col] = s * ap + c * aq;
      }
      __syncthreads();
      // columns p, q of every pair: A <- A J
      for (int e = tid; e < npairs * M; e += 256) {
        const int k = e / M, row = e % M;
        const int p = sp[k], q = sq[k];
        if (q >= M) continue;
        const float c = sc[k], s = ss[k];
        const float ap = A[(int64_t)row * M + p], aq = A[(int64_t)row * M + q];
        A[(int64_t)row * M + p] = c * ap - s * aq;
        A[(int64_t)row * M + q] = s * ap + c * aq;
      }
      __syncthreads();
    }
  }
  // eigenvalues = diagonal, by decreasing value (rank by counting; ties by index)
  for (int i = tid; i < M; i += 256) sdiag[i] = A[(int64_t)i * M + i];
  __syncthreads();
  for (int i = tid; i < M; i += 256) {
    const float d = sdiag[i];
    int rank = 0;
    for (int k = 0; k < M; ++k) rank += (sdiag[k] > d) || (sdiag[k] == d && k < i);
    a.eig[(a.bh0 + lbh) * M + rank] = d;
  }
}

}  // namespace flarepp

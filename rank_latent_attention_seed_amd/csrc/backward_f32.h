// Backward of the route in float32 vector arithmetic: the gradients dS, dK,
// dV of a scalar loss, given dY.  For one SDPA application
// O = SDPA(Q, K, V, s) with P_ij = softmax_j(s <Q_i, K_j>) and upstream dO:
//     dV_j += sum_i P_ij dO_i,        dP_ij = <dO_i, V_j>,
//     dL_ij  = P_ij (dP_ij - delta_i),  delta_i = sum_j P_ij dP_ij = <dO_i, O_i>,
//     dQ_i  += s sum_j dL_ij K_j,     dK_j += s sum_i dL_ij Q_i
// (the chain rule through the SDPA form of the FLARE summary, "Основной
// механизм FLARE"), taken through the three stages in reverse: the decode
// (queries = tokens, keys = Qd, values = Z), the encode (queries = Qd), the
// seed encode (queries = S).  Qd feeds both the encode (as query) and the
// decode (as key), so its gradient collects both before the seed encode.
//
// Softmax weights are recomputed from the forward's log-sum-exp statistics
// (log2 units, t = c <q, k> with c = s log2 e, P = exp2(t - A)).  Each stage
// runs two kernels:
//   * a token pass: one thread per token, the M latent rows staged in LDS,
//     accumulating the token's dK (and dV) in registers;
//   * a latent pass: one thread per latent, the tokens of one split staged in
//     LDS, accumulating the latent's gradients; splits are summed by
//     bwd_reduce.
#pragma once

#include "common.h"

namespace flarepp {

// Latent-side float32 rows of the launch's heads are [G][M][D] (head lbh's
// rows start at lbh * M * D), per-latent scalars [G][Mp]; the query rows are
// addressed like the forward's operands (b * q_sb + h * q_sh - q_off), which
// also covers the seed block of stage 1 (q_sb = 0, q_sh = 0 or M * D).
struct BwdTokArgs {
  const float* q;      // latent query rows of this stage (Qd for the decode: its keys)
  int64_t q_sb, q_sh, q_off;  // (b, h)'s rows start at b*q_sb + h*q_sh - q_off
  const float* lat2;   // decode: Z rows; encode: dO rows ([G][M][D])
  const float* lse;    // encode: per-latent log-sum-exp A_m ([G][Mp]); decode: unused
  const float* delta;  // encode: per-latent <dO_m, O_m> ([G][Mp]); decode: unused
  const float* K;      // B x H x N x D
  const float* V;      // encode: values; decode: unused
  const float* dY;     // decode: upstream dY (B x H x N x D); encode: unused
  float* dK;           // B x H x N x D
  float* dV;           // encode: B x H x N x D; decode: unused
  float* tlse;         // decode: per-token A_n ([G][N]), written
  float* tdelta;       // decode: per-token <dY_n, Y_n> ([G][N]), written
  int H, N, M, Mp;
  int64_t bh0;
  float c, s;
  int acc_dk, acc_dv;  // add into dK / dV (else overwrite)
};

// Maximum latents whose two D-float rows fit the token kernels' LDS.
constexpr int kBwdMaxM = 256;

// Decode token pass: for token n with query k_n over the latents (keys Qd,
// values Z), recompute A_n and Y_n, then
//   dK_n = s sum_m P_nm (<dY_n, Z_m> - <dY_n, Y_n>) Qd_m.
// The shift is the Cauchy-Schwarz bound c ||k_n|| max ||Qd_m|| when it keeps
// every exponent within [-100, 0]; else an exact max pass over the latents.
template <int D>
__global__ __launch_bounds__(256) void bwd_decode_tokens(BwdTokArgs a) {
  __shared__ float sQ[kBwdMaxM * D];
  __shared__ float sZ[kBwdMaxM * D];
  __shared__ float sQmax[8];
  const int tid = threadIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const float* qp = a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off;
  const float* zp = a.lat2 + lbh * (int64_t)a.M * D;
  float qn2 = 0.0f;
  for (int e = tid; e < a.M * D; e += 256) {
    const float x = qp[e];
    sQ[e] = x;
    sZ[e] = zp[e];
  }
  __syncthreads();
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
  const int64_t row = (bh * (int64_t)a.N + n) * D;
  float k[D], g[D];
  float kn2 = 0.0f;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    k[d] = a.K[row + d];
    g[d] = a.dY[row + d];
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
  // A_n and Y_n
  float lam = 0.0f, y[D];
#pragma unroll
  for (int d = 0; d < D; ++d) y[d] = 0.0f;
  for (int m = 0; m < a.M; ++m) {
    const float p = exp2f(logit(m) - mu);
    lam += p;
#pragma unroll
    for (int d = 0; d < D; ++d) y[d] = fmaf(p, sZ[m * D + d], y[d]);
  }
  const float A = mu + log2f(lam);
  float delta = 0.0f;
#pragma unroll
  for (int d = 0; d < D; ++d) delta = fmaf(g[d], y[d] / lam, delta);
  // dK_n
  float dk[D];
#pragma unroll
  for (int d = 0; d < D; ++d) dk[d] = 0.0f;
  for (int m = 0; m < a.M; ++m) {
    const float p = exp2f(logit(m) - A);
    float dp = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) dp = fmaf(g[d], sZ[m * D + d], dp);
    const float dl = a.s * p * (dp - delta);
#pragma unroll
    for (int d = 0; d < D; ++d) dk[d] = fmaf(dl, sQ[m * D + d], dk[d]);
  }
#pragma unroll
  for (int d = 0; d < D; ++d) a.dK[row + d] = a.acc_dk ? a.dK[row + d] + dk[d] : dk[d];
  a.tlse[lbh * (int64_t)a.N + n] = A;
  a.tdelta[lbh * (int64_t)a.N + n] = delta;
}

// Encode token pass (stages 1 and 2): for token n,
//   dV_n += sum_m P_mn dO_m,   dK_n += s sum_m P_mn (<dO_m, V_n> - delta_m) Q_m
// with P_mn = exp2(c <Q_m, K_n> - A_m).
template <int D>
__global__ __launch_bounds__(256) void bwd_encode_tokens(BwdTokArgs a) {
  __shared__ float sQ[kBwdMaxM * D];
  __shared__ float sG[kBwdMaxM * D];
  __shared__ float sA[kBwdMaxM];
  __shared__ float sDel[kBwdMaxM];
  const int tid = threadIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const float* qp = a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off;
  const float* gp = a.lat2 + lbh * (int64_t)a.M * D;
  for (int e = tid; e < a.M * D; e += 256) {
    sQ[e] = qp[e];
    sG[e] = gp[e];
  }
  for (int m = tid; m < a.M; m += 256) {
    sA[m] = a.lse[lbh * a.Mp + m];
    sDel[m] = a.delta[lbh * a.Mp + m];
  }
  __syncthreads();
  const int n = blockIdx.x * 256 + tid;
  if (n >= a.N) return;
  const int64_t row = (bh * (int64_t)a.N + n) * D;
  float k[D], v[D], dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    k[d] = a.K[row + d];
    v[d] = a.V[row + d];
    dk[d] = 0.0f;
    dv[d] = 0.0f;
  }
  for (int m = 0; m < a.M; ++m) {
    float t = 0.0f, dp = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      t = fmaf(sQ[m * D + d], k[d], t);
      dp = fmaf(sG[m * D + d], v[d], dp);
    }
    const float p = exp2f(a.c * t - sA[m]);
    const float dl = a.s * p * (dp - sDel[m]);
#pragma unroll
    for (int d = 0; d < D; ++d) {
      dv[d] = fmaf(p, sG[m * D + d], dv[d]);
      dk[d] = fmaf(dl, sQ[m * D + d], dk[d]);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    a.dK[row + d] = a.acc_dk ? a.dK[row + d] + dk[d] : dk[d];
    a.dV[row + d] = a.acc_dv ? a.dV[row + d] + dv[d] : dv[d];
  }
}

struct BwdLatArgs {
  const float* q;      // latent rows of this stage (queries; Qd for the decode)
  int64_t q_sb, q_sh, q_off;
  const float* lat2;   // decode: Z rows; encode: dO rows ([G][M][D])
  const float* lse;    // encode: [G][Mp]
  const float* delta;  // encode: [G][Mp]
  const float* K;
  const float* V;      // encode: values
  const float* dY;     // decode: upstream dY
  const float* tlse;   // decode: per-token A_n ([G][N])
  const float* tdelta; // decode: per-token delta_n ([G][N])
  float* part;         // [G][Mp][J][R] partial sums (R = 2D decode, D encode)
  int H, N, M, Mp, J, chunk;
  int64_t bh0;
  float c, s;
};

// Latent passes, one thread per latent, over one split of the tokens staged
// in LDS 64 at a time.
//   decode:  dZ_m  += sum_n P_nm dY_n,   dQd_m += s sum_n P_nm (<dY_n, Z_m> - delta_n) K_n
//   encode:  dQ_m  += s sum_n P_mn (<dO_m, V_n> - delta_m) K_n
template <int D, bool DECODE>
__global__ __launch_bounds__(256) void bwd_latents(BwdLatArgs a) {
  constexpr int TN = 64;
  constexpr int R = DECODE ? 2 * D : D;
  __shared__ float sK[TN * D];
  __shared__ float sW[TN * D];  // decode: dY rows; encode: V rows
  __shared__ float sA[TN];
  __shared__ float sDel[TN];
  const int tid = threadIdx.x;
  const int j = blockIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const int m = blockIdx.z * 256 + tid;
  const bool real = m < a.M;
  const int n0 = j * a.chunk, n1 = min(a.N, n0 + a.chunk);

  const float* qp = a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off + (int64_t)m * D;
  const float* gp = a.lat2 + (lbh * (int64_t)a.M + m) * D;
  float q[D], w[D], g1[D], g2[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = real ? qp[d] : 0.0f;
    w[d] = real ? gp[d] : 0.0f;  // decode: Z_m; encode: dO_m
    g1[d] = 0.0f;
    g2[d] = 0.0f;
  }
  const float Am = (!DECODE && real) ? a.lse[lbh * a.Mp + m] : 0.0f;
  const float Dm = (!DECODE && real) ? a.delta[lbh * a.Mp + m] : 0.0f;

  const float* Kp = a.K + bh * (int64_t)a.N * D;
  const float* Wp = (DECODE ? a.dY : a.V) + bh * (int64_t)a.N * D;
  for (int tb = n0; tb < n1; tb += TN) {
    const int cnt = min(TN, n1 - tb);
    __syncthreads();
    for (int e = tid; e < cnt * D; e += 256) {
      sK[e] = Kp[(int64_t)tb * D + e];
      sW[e] = Wp[(int64_t)tb * D + e];
    }
    if (DECODE)
      for (int e = tid; e < cnt; e += 256) {
        sA[e] = a.tlse[lbh * (int64_t)a.N + tb + e];
        sDel[e] = a.tdelta[lbh * (int64_t)a.N + tb + e];
      }
    __syncthreads();
    for (int n = 0; n < cnt; ++n) {
      float t = 0.0f, dp = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        t = fmaf(q[d], sK[n * D + d], t);
        dp = fmaf(w[d], sW[n * D + d], dp);
      }
      const float p = exp2f(a.c * t - (DECODE ? sA[n] : Am));
      const float dl = a.s * p * (dp - (DECODE ? sDel[n] : Dm));
#pragma unroll
      for (int d = 0; d < D; ++d) {
        g1[d] = fmaf(dl, sK[n * D + d], g1[d]);               // dQd (decode) / dQ (encode)
        if (DECODE) g2[d] = fmaf(p, sW[n * D + d], g2[d]);   // dZ
      }
    }
  }
  if (!real) return;
  float* rec = a.part + ((lbh * (int64_t)a.Mp + m) * a.J + j) * R;
#pragma unroll
  for (int d = 0; d < D; ++d) rec[d] = g1[d];
  if (DECODE)
#pragma unroll
    for (int d = 0; d < D; ++d) rec[D + d] = g2[d];
}

// Sums of the split partials.  Per-head mode (seed_blocks == 0): thread
// (lbh, m, d) writes out[lbh][m][d] = sum_j part[lbh][m][j][field0 + d]
// (+ add_to[lbh][m][d]), rows [G][M][D]; with dot_with it also writes
// delta[lbh][m] = <out_m, dot_with_m>.  Seed mode (seed_blocks = 1 or H):
// thread (k, m, d) adds the sums of every launch head whose seed block is k
// into out[k][m][d] (the caller zeroes out once; launches run in order).
struct BwdReduceArgs {
  const float* part;
  int J, R, field0, M, Mp, G, H;
  int64_t bh0;
  const float* add_to;
  float* out;
  const float* dot_with;
  float* delta;
  int seed_blocks;
};

template <int D>
__global__ __launch_bounds__(256) void bwd_reduce(BwdReduceArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int d = (int)(idx % D);
  const int64_t r = idx / D;
  const bool seeds = a.seed_blocks > 0;
  const int64_t rows = (int64_t)(seeds ? a.seed_blocks : a.G) * a.M;
  const bool live = r < rows;
  const int blk = live ? (int)(r / a.M) : 0;
  const int m = live ? (int)(r % a.M) : 0;
  float acc = 0.0f;
  if (live) {
    for (int lbh = seeds ? 0 : blk; lbh < (seeds ? a.G : blk + 1); ++lbh) {
      if (seeds && a.seed_blocks > 1 && (int)((a.bh0 + lbh) % a.H) != blk) continue;
      const float* p = a.part + ((lbh * (int64_t)a.Mp + m) * a.J) * a.R + a.field0 + d;
      for (int j = 0; j < a.J; ++j) acc += p[(int64_t)j * a.R];
    }
    if (a.add_to) acc += a.add_to[r * D + d];
  }
  // a row's D elements are D adjacent lanes
  float dd = 0.0f;
  if (a.dot_with) {
    dd = live ? acc * a.dot_with[r * D + d] : 0.0f;
#pragma unroll
    for (int off = D / 2; off >= 1; off >>= 1) dd += __shfl_xor(dd, off);
  }
  if (!live) return;
  if (seeds)
    a.out[r * D + d] += acc;
  else
    a.out[r * D + d] = acc;
  if (a.dot_with && d == 0) a.delta[(int64_t)blk * a.Mp + m] = dd;
}

// dst[i] = 0 for i < n (float32).
__global__ __launch_bounds__(256) void fill_zero(float* dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = 0.0f;
}

}  // namespace flarepp

// Float32 path: the same three SDPA stages in float32 vector arithmetic.
// It targets accuracy (relative error ~1e-6) rather than matrix-core
// throughput, and writes the same split partial records as the bf16 encode so
// that the merge kernel is shared.
#pragma once

#include "common.h"

namespace flarepp {

// Split-N encode, one latent per thread: online softmax over the split's
// tokens (FLARE summary, "Основной механизм FLARE", encode step).
struct EncodeF32Args {
  const float* q;      // query rows (M x D per block)
  int64_t q_sb, q_sh, q_off;  // element offset of (b, h)'s rows: b*q_sb + h*q_sh - q_off
  const float* K;
  const float* V;
  float* part;         // [G][Mp][J][D + 4]
  int H, N, M, Mp, J, chunk;
  int64_t bh0;
  float c;             // scale * log2(e)
};

template <int D>
__global__ __launch_bounds__(256) void encode_split_f32(EncodeF32Args a) {
  constexpr int TN = 64;
  __shared__ float sK[TN * D];
  __shared__ float sV[TN * D];
  const int tid = threadIdx.x;
  const int j = blockIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const int m = blockIdx.z * 256 + tid;
  const int n0 = j * a.chunk, n1 = min(a.N, n0 + a.chunk);
  const bool real = m < a.M;

  float q[D];
  const float* qp = a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off + (int64_t)m * D;
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = real ? qp[d] * a.c : 0.0f;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.0f;
  float mu = -INFINITY, lam = 0.0f;

  const float* Kp = a.K + bh * (int64_t)a.N * D;
  const float* Vp = a.V + bh * (int64_t)a.N * D;
  for (int tb = n0; tb < n1; tb += TN) {
    const int cnt = min(TN, n1 - tb);
    __syncthreads();
    for (int e = tid; e < cnt * D; e += 256) {
      sK[e] = Kp[(int64_t)tb * D + e];
      sV[e] = Vp[(int64_t)tb * D + e];
    }
    __syncthreads();
    for (int n = 0; n < cnt; ++n) {
      float t = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) t = fmaf(q[d], sK[n * D + d], t);
      if (t > mu) {
        const float al = exp2f(mu - t);
        lam *= al;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= al;
        mu = t;
      }
      const float p = exp2f(t - mu);
      lam += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, sV[n * D + d], acc[d]);
    }
  }
  if (m < a.Mp) {
    float* rec = a.part + ((lbh * a.Mp + m) * (int64_t)a.J + j) * Part<D>::kStride;
#pragma unroll
    for (int d = 0; d < D; ++d) rec[d] = real ? acc[d] : 0.0f;
    rec[D] = real ? lam : 1.0f;
    rec[D + 1] = real ? mu : 0.0f;
  }
}

// Decode, one token per thread, exact max over the latents then the weighted
// sum (FLARE summary, "Основной механизм FLARE", decode step).
struct DecodeF32Args {
  const float* qd;     // Qd rows: (b, h)'s M x D block at b*q_sb + h*q_sh - q_off
  int64_t q_sb, q_sh, q_off;
  const float* z;      // Z rows: (b, h)'s block at b*z_sb + h*z_sh - z_off
  int64_t z_sb, z_sh, z_off;
  const float* K;
  float* Y;
  int H, N, M;
  int64_t bh0;
  float c;
};

template <int D>
__global__ __launch_bounds__(256) void decode_f32(DecodeF32Args a) {
  extern __shared__ float sm[];  // [M][D] c*Qd, then [M][D] Z
  float* sQ = sm;
  float* sZ = sm + (int64_t)a.M * D;
  const int tid = threadIdx.x;
  const int64_t bh = a.bh0 + blockIdx.y;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const int64_t qo = (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off;
  const int64_t zo = (int64_t)b * a.z_sb + (int64_t)h * a.z_sh - a.z_off;
  for (int e = tid; e < a.M * D; e += 256) {
    sQ[e] = a.qd[qo + e] * a.c;
    sZ[e] = a.z[zo + e];
  }
  __syncthreads();
  const int n = blockIdx.x * 256 + tid;
  if (n >= a.N) return;
  const float* kp = a.K + (bh * a.N + n) * (int64_t)D;
  float k[D];
#pragma unroll
  for (int d = 0; d < D; ++d) k[d] = kp[d];
  float mx = -INFINITY;
  for (int m = 0; m < a.M; ++m) {
    float t = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) t = fmaf(sQ[m * D + d], k[d], t);
    mx = fmaxf(mx, t);
  }
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.0f;
  float lam = 0.0f;
  for (int m = 0; m < a.M; ++m) {
    float t = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) t = fmaf(sQ[m * D + d], k[d], t);
    const float p = exp2f(t - mx);
    lam += p;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(p, sZ[m * D + d], acc[d]);
  }
  const float inv = 1.0f / lam;
  float* yp = a.Y + (bh * a.N + n) * (int64_t)D;
#pragma unroll
  for (int d = 0; d < D; ++d) yp[d] = acc[d] * inv;
}

}  // namespace flarepp

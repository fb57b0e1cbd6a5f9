// Cross-workgroup merge of split-N softmax partials, and the query-operand
// preparation used by the next stage.
//
// A split j of the tokens leaves, per latent m, its running max mu_j (log2
// units), the sum lambda_j of its weights exp2(t - mu_j) and the matching
// unnormalised accumulator acc_j.  The exact softmax over all tokens is
//     O_m = sum_j 2^(mu_j - mu) acc_j / sum_j 2^(mu_j - mu) lambda_j,
//     mu  = max_j mu_j,
// the same combination of "latent outputs and softmax statistics" the pages
// use to join token shards across devices (French technical summary,
// "Contributions Clés", context parallelism).  The merged rows are written as
// float32 (the caller's Qd or Z) and, for the next stage, as bf16 operands:
// c * row as a hi/lo pair (hi = bf16(x), lo = bf16(x - hi)), the unscaled row
// as bf16, and the row's Euclidean norm.
#pragma once

#include "common.h"

namespace flarepp {

// Buffers marked [G] are indexed by the launch-local head lbh = blockIdx.y;
// the caller's output by the global (b, h) = bh0 + lbh.
struct MergeArgs {
  float* part;         // [G][Mp][J][D + 4] (records recomputed by refit_record are written back)
  int J, Mp, M;
  int64_t bh0;
  float* out;          // [BH][M][D] float32 (the caller's Qd or Z), or null
  float* outl;         // [G][M][D] float32 staging copy, or null
  __bf16* op_hi;       // [G][Mp][D] bf16(c * row), or null
  __bf16* op_lo;       // [G][Mp][D] bf16(c * row - hi), or null
  __bf16* op_zt;       // [G][D][Mp] bf16(row), transposed, or null
  float* qnorm;        // [G][Mp] ||row||, or null
  const float* knorm;  // [G][Jk] squared key norms per split of a seed encode, or null
  int Jk;
  float* bias;         // [G][Mp] bound |c| ||row|| max||K|| for the next encode (+inf if unsafe), or null
  float c;
  float* lse;          // [G][Mp] log-sum-exp of the row's softmax, log2 units (mu + log2 lambda), or null
  // Record mode (rec_out non-null): instead of the rows, write each row's
  // combined record -- the unnormalised (acc, lambda, mu) -- to slot rec_slot
  // of rec_out [BH][Mp][rec_nslots][D + 4] (a token shard's share of the
  // stage, for a later merge over the shards).
  float* rec_out;
  int rec_slot, rec_nslots;
  // The encode whose records are merged, for refit_record (fK null: none is
  // recomputed): its query operand rows (bf16 hi/lo of c * Q, the rows of
  // (b, h) at b*fq_sb + h*fq_sh - fq_off), K, V and token splits.
  const __bf16* fq_hi;
  const __bf16* fq_lo;
  const __bf16* fq_seed;  // or the unscaled seed rows [.][M][D] (EncodeArgs::q_seed), scaled by fq_c
  float fq_c;
  int64_t fq_sb, fq_sh, fq_off;
  const __bf16* fK;
  const __bf16* fV;
  int H, N, chunk;
};

// A record whose sum is not finite comes from an encode whose fp16 weights
// overflowed in a tile that skipped the running-max check (encode_bf16.h,
// Pv); it is recomputed here, for one latent m and one split j, with the
// encode's arithmetic in float32 on the VALU and no rounding of the weights:
// t_n = <c Q_m, K_n> (log2 units), mu = max t_n, lambda = sum 2^(t_n - mu),
// acc = sum 2^(t_n - mu) V_n.  Slow (one thread walks the split), and taken
// only for inputs whose scores jump far past the running max within a tile.
template <int D>
__device__ __forceinline__ void refit_record(const MergeArgs& a, int64_t bh, int m, int j, float* rec) {
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const int64_t qo = (int64_t)b * a.fq_sb + (int64_t)h * a.fq_sh - a.fq_off + (int64_t)m * D;
  // the encode's query: the exact seed row (zero past M), its products
  // scaled by c, or the hi + lo operand of c Q
  float q[D];
  const float qs = a.fq_seed ? a.fq_c : 1.0f;
#pragma unroll
  for (int d = 0; d < D; ++d)
    q[d] = a.fq_seed ? (m < a.M ? (float)a.fq_seed[qo + d] : 0.0f) : (float)a.fq_hi[qo + d] + (float)a.fq_lo[qo + d];
  const int n0 = j * a.chunk, n1 = min(a.N, n0 + a.chunk);
  const __bf16* Kp = a.fK + bh * (int64_t)a.N * D;
  const __bf16* Vp = a.fV + bh * (int64_t)a.N * D;
  auto logit = [&](int n) {
    float t = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) t = fmaf(q[d], (float)Kp[(int64_t)n * D + d], t);
    return qs * t;
  };
  float mu = -INFINITY;
  for (int n = n0; n < n1; ++n) mu = fmaxf(mu, logit(n));
  float lam = 0.0f, acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.0f;
  for (int n = n0; n < n1; ++n) {
    const float w = exp2f(logit(n) - mu);
    lam += w;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(w, (float)Vp[(int64_t)n * D + d], acc[d]);
  }
#pragma unroll
  for (int d = 0; d < D; ++d) rec[d] = acc[d];
  rec[D] = lam;
  rec[D + 1] = mu;
}

// Largest exponent span (log2 units) a bound-shifted softmax may cover: with
// every exponent in [-100, 0] the largest weight is >= 2^-100, far above the
// float32 / bf16 normal range floor 2^-126.
constexpr float kBoundSpan = 100.0f;

// Reductions over the T threads that share a latent row (T a power of two,
// the group aligned within one wave).
template <int T>
__device__ __forceinline__ float group_sum(float x) {
  if (T == 64) return wave_sum(x);
#pragma unroll
  for (int off = T / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}
template <int T>
__device__ __forceinline__ float group_max(float x) {
  if (T == 64) return wave_max(x);
#pragma unroll
  for (int off = T / 2; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// Sums over the 64 lanes of a wave of 32 values per lane, every lane getting
// all 32 sums: two halving steps (each lane pair swaps half its values
// through a permlane swap and keeps the sums of the other half: 16, then 8
// values left, lane l holding elements 8 (l / 16) .. + 7 summed over the
// lanes l, l ^ 16, l ^ 32, l ^ 48), an all-reduce of those 8 within each
// 16-lane row (DPP), and a gather of the four rows' results through the same
// swaps: about 100 VALU instructions where 32 separate wave sums take ~300.
__device__ __forceinline__ void wave_sum32(float (&v)[32]) {
  auto f = [](uint32_t u) { return __uint_as_float(u); };
  auto u = [](float x) { return __float_as_uint(x); };
  float h[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // lanes < 32 keep element i, lanes >= 32 element i + 16
    const auto t = __builtin_amdgcn_permlane32_swap(u(v[i]), u(v[i + 16]), false, false);
    h[i] = f(t[0]) + f(t[1]);
  }
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // then rows 0 / 2 keep h[i], rows 1 / 3 h[i + 8]
    const auto t = __builtin_amdgcn_permlane16_swap(u(h[i]), u(h[i + 8]), false, false);
    r[i] = f(t[0]) + f(t[1]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // row r: element 8 r + i, summed over its 16 lanes
    r[i] += dpp<0xB1>(r[i]);
    r[i] += dpp<0x4E>(r[i]);
    r[i] += dpp<0x124>(r[i]);
    r[i] += dpp<0x128>(r[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const auto p = __builtin_amdgcn_permlane16_swap(u(r[i]), u(r[i]), false, false);  // rows 2k, 2k + 1
    const auto a = __builtin_amdgcn_permlane32_swap(p[0], p[0], false, false);        // rows 0, 2
    const auto b = __builtin_amdgcn_permlane32_swap(p[1], p[1], false, false);        // rows 1, 3
    v[i] = f(a[0]);
    v[16 + i] = f(a[1]);
    v[8 + i] = f(b[0]);
    v[24 + i] = f(b[1]);
  }
}

// One latent row per group of T threads (T = 64 for many splits: one row per
// wave).  Thread q of a row folds splits q, q + T, ...: a first sweep over
// the maxima only, then the weighted sums, each unrolled so that its loads are
// in flight together; the row's records are contiguous, so a wave's loads
// are coalesced.
template <int D, int T>
__global__ __launch_bounds__(256) void merge_partials(MergeArgs a) {
  constexpr int PS = Part<D>::kStride;
  constexpr int RPB = 256 / T;
  const int tid = threadIdx.x;
  const int r = tid / T, q = tid % T;
  const int m = blockIdx.x * RPB + r;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const bool row_ok = m < a.Mp;
  float* base = a.part + ((lbh * a.Mp + (row_ok ? m : 0)) * (int64_t)a.J) * PS;
  float mx, den, x[D];
  if (D == 32 && T == 64 && a.J <= 64) {
    // one record per lane, read in one pass (a record whose sum is not finite
    // is recomputed, then read again), weighted, then reduced by wave_sum32
    const bool has = row_ok && q < a.J;
    float* rec = base + (int64_t)q * PS;
    f32x4 rv[D / 4], tail = f32x4{0.f, -INFINITY, 0.f, 0.f};
#pragma unroll
    for (int d4 = 0; d4 < D / 4; ++d4) rv[d4] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto load = [&]() {
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4) rv[d4] = *reinterpret_cast<const f32x4*>(rec + 4 * d4);
      tail = *reinterpret_cast<const f32x4*>(rec + D);
    };
    if (has) {
      load();
      if (a.fK && !(tail[0] <= 3.0e38f)) {
        refit_record<D>(a, bh, m, q, rec);
        load();
      }
    }
    mx = wave_max(tail[1]);
    const float w = has ? fast_exp2(tail[1] - mx) : 0.0f;
    den = wave_sum(w * tail[0]);
#pragma unroll
    for (int d4 = 0; d4 < D / 4; ++d4)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * d4 + e] = w * rv[d4][e];
    if constexpr (D == 32) wave_sum32(x);
  } else {
    if (a.fK && row_ok)
      for (int jj = q; jj < a.J; jj += T)
        if (!(base[(int64_t)jj * PS + D] <= 3.0e38f)) refit_record<D>(a, bh, m, jj, base + (int64_t)jj * PS);

    mx = -INFINITY;
#pragma unroll 8
    for (int jj = q; jj < a.J; jj += T) mx = fmaxf(mx, base[(int64_t)jj * PS + D + 1]);
    mx = group_max<T>(mx);

    den = 0.0f;
    f32x4 num[D / 4];
#pragma unroll
    for (int d4 = 0; d4 < D / 4; ++d4) num[d4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int jj = q; jj < a.J; jj += T) {
      const float* rec = base + (int64_t)jj * PS;
      const f32x4 tl = *reinterpret_cast<const f32x4*>(rec + D);
      const float w = fast_exp2(tl[1] - mx);
      den += w * tl[0];
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4) num[d4] += w * *reinterpret_cast<const f32x4*>(rec + 4 * d4);
    }
    den = group_sum<T>(den);
#pragma unroll
    for (int d4 = 0; d4 < D / 4; ++d4)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * d4 + e] = group_sum<T>(num[d4][e]);
  }

  if (a.rec_out) {
    if (!row_ok) return;
    float* o = a.rec_out + ((bh * a.Mp + m) * (int64_t)a.rec_nslots + a.rec_slot) * PS;
    for (int d = q; d < D; d += T) {
      float v = x[0];
#pragma unroll
      for (int e = 1; e < D; ++e) v = (d == e) ? x[e] : v;
      o[d] = v;
    }
    if (q == 0) *reinterpret_cast<f32x4*>(o + D) = f32x4{den, mx, 0.0f, 0.0f};
    return;
  }

  const bool real = m < a.M;
  const float inv = 1.0f / den;
  float n2 = 0.0f;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    x[d] = real ? x[d] * inv : 0.0f;
    n2 += x[d] * x[d];
  }
  const float nrm = sqrtf(n2);

  float kmax2 = 0.0f;
  if (a.bias && a.knorm) {
    const float* kn = a.knorm + lbh * a.Jk;
    for (int jj = q; jj < a.Jk; jj += T) kmax2 = fmaxf(kmax2, kn[jj]);
    kmax2 = group_max<T>(kmax2);
  }
  if (!row_ok) return;

  // every thread of the row holds the whole row: thread q writes elements q, q + T, ...
  const int64_t orow = (lbh * a.Mp + m) * D;
  constexpr int PER = (D + T - 1) / T;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int d = q + k * T;
    if (d >= D) break;
    float v = x[0];
#pragma unroll
    for (int e = 1; e < D; ++e) v = (d == e) ? x[e] : v;
    if (a.out && real) a.out[(bh * a.M + m) * D + d] = v;
    if (a.outl && real) a.outl[(lbh * a.M + m) * D + d] = v;
    if (a.op_hi) {
      const float xs = v * a.c;
      const __bf16 hi = (__bf16)xs;
      a.op_hi[orow + d] = hi;
      if (a.op_lo) a.op_lo[orow + d] = (__bf16)(xs - (float)hi);
    }
    if (a.op_zt) a.op_zt[(lbh * D + d) * (int64_t)a.Mp + m] = (__bf16)v;
  }
  if (q == 0) {
    if (a.lse) a.lse[lbh * a.Mp + m] = mx + log2f(den);
    if (a.qnorm) a.qnorm[lbh * a.Mp + m] = nrm;
    if (a.bias) {
      float bnd = INFINITY;
      if (a.knorm) {
        bnd = fabsf(a.c) * nrm * sqrtf(kmax2) * (1.0f + 1.0f / 4096.0f);
        if (!(2.0f * bnd <= kBoundSpan)) bnd = INFINITY;
      }
      a.bias[lbh * a.Mp + m] = bnd;
    }
  }
}

// The same merge with one latent row per 256-thread workgroup, for many
// splits (128 < J <= 512): thread q holds records q and q + 256 in registers,
// so the records are read once; the maxima, then the weighted sums, are
// reduced over the workgroup (DPP within waves, LDS across the four).
// Wave 0 finishes the row: lane d < D owns element d.
template <int D>
__global__ __launch_bounds__(256) void merge_rows256(MergeArgs a) {
  constexpr int PS = Part<D>::kStride;
  constexpr int NV = PS / 4;  // float4s per record
  __shared__ float sRed[4][D + 1];
  __shared__ float sMax[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = blockIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  float* base = a.part + ((lbh * a.Mp + m) * (int64_t)a.J) * PS;

  const bool h0 = tid < a.J, h1 = tid + 256 < a.J;
  if (a.fK) {  // records with a non-finite sum: recompute before reading (see refit_record)
    if (h0 && !(base[(int64_t)tid * PS + D] <= 3.0e38f)) refit_record<D>(a, bh, m, tid, base + (int64_t)tid * PS);
    if (h1 && !(base[(int64_t)(tid + 256) * PS + D] <= 3.0e38f))
      refit_record<D>(a, bh, m, tid + 256, base + (int64_t)(tid + 256) * PS);
  }
  f32x4 r0[NV], r1[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    r0[v] = h0 ? *reinterpret_cast<const f32x4*>(base + (int64_t)tid * PS + 4 * v) : f32x4{0.f, 0.f, 0.f, 0.f};
    r1[v] = h1 ? *reinterpret_cast<const f32x4*>(base + (int64_t)(tid + 256) * PS + 4 * v)
               : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // record tail: lambda at D, mu at D + 1
  const float mu0 = h0 ? r0[D / 4][1] : -INFINITY, mu1 = h1 ? r1[D / 4][1] : -INFINITY;
  float mx = wave_max(fmaxf(mu0, mu1));
  if (lane == 0) sMax[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(sMax[0], sMax[1]), fmaxf(sMax[2], sMax[3]));
  const float w0 = h0 ? fast_exp2(mu0 - mx) : 0.0f, w1 = h1 ? fast_exp2(mu1 - mx) : 0.0f;
#pragma unroll
  for (int v = 0; v < D / 4; ++v) {
    const f32x4 y = w0 * r0[v] + w1 * r1[v];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float t = wave_sum(y[e]);
      if (lane == 0) sRed[wave][4 * v + e] = t;
    }
  }
  {
    const float t = wave_sum(w0 * r0[D / 4][0] + w1 * r1[D / 4][0]);
    if (lane == 0) sRed[wave][D] = t;
  }
  float kmax2 = 0.0f;
  if (a.bias && a.knorm && wave == 0) {
    const float* kn = a.knorm + lbh * a.Jk;
    for (int jj = lane; jj < a.Jk; jj += 64) kmax2 = fmaxf(kmax2, kn[jj]);
    kmax2 = wave_max(kmax2);
  }
  __syncthreads();
  if (wave != 0) return;

  const bool real = m < a.M;
  const float den = sRed[0][D] + sRed[1][D] + sRed[2][D] + sRed[3][D];
  const int d = lane < D ? lane : 0;
  if (a.rec_out) {  // record mode (see MergeArgs)
    float* o = a.rec_out + ((bh * a.Mp + m) * (int64_t)a.rec_nslots + a.rec_slot) * PS;
    if (lane < D) o[lane] = sRed[0][d] + sRed[1][d] + sRed[2][d] + sRed[3][d];
    if (lane == 0) *reinterpret_cast<f32x4*>(o + D) = f32x4{den, mx, 0.0f, 0.0f};
    return;
  }
  float x = (sRed[0][d] + sRed[1][d] + sRed[2][d] + sRed[3][d]) / den;
  if (!real || lane >= D) x = 0.0f;
  const float nrm = sqrtf(wave_sum(x * x));
  if (lane < D) {
    const int64_t orow = (lbh * a.Mp + m) * D;
    if (a.out && real) a.out[(bh * a.M + m) * D + d] = x;
    if (a.outl && real) a.outl[(lbh * a.M + m) * D + d] = x;
    if (a.op_hi) {
      const float xs = x * a.c;
      const __bf16 hi = (__bf16)xs;
      a.op_hi[orow + d] = hi;
      if (a.op_lo) a.op_lo[orow + d] = (__bf16)(xs - (float)hi);
    }
    if (a.op_zt) a.op_zt[(lbh * D + d) * (int64_t)a.Mp + m] = (__bf16)x;
  }
  if (lane == 0) {
    if (a.lse) a.lse[lbh * a.Mp + m] = mx + log2f(den);
    if (a.qnorm) a.qnorm[lbh * a.Mp + m] = nrm;
    if (a.bias) {
      float bnd = INFINITY;
      if (a.knorm) {
        bnd = fabsf(a.c) * nrm * sqrtf(kmax2) * (1.0f + 1.0f / 4096.0f);
        if (!(2.0f * bnd <= kBoundSpan)) bnd = INFINITY;
      }
      a.bias[lbh * a.Mp + m] = bnd;
    }
  }
}

// Operands from a caller's rows (float32 or bf16): nblk blocks of M x D rows,
// block k starting at element src_off + k * src_blk -> [nblk][Mp][D] bf16 hi/lo
// of c * row, [nblk][D][Mp] bf16 of the row (transposed) and row norms; rows
// M..Mp-1 are zero.
struct PrepArgs {
  const void* src;
  int src_bf16;
  int64_t src_off, src_blk;
  int nblk, M, Mp;
  __bf16* op_hi;
  __bf16* op_lo;
  __bf16* op_zt;
  float* qnorm;
  float c;
};

// One thread per element: a row's D elements are D adjacent lanes, whose
// squared sum gives the row norm.
template <int D>
__global__ __launch_bounds__(256) void prep_rows(PrepArgs a) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)a.nblk * a.Mp;
  const int64_t idx = e / D;  // row (over all blocks)
  const int d = (int)(e % D);
  const bool live = idx < rows;  // whole rows are live or not (D divides 64)
  const int64_t blk = live ? idx / a.Mp : 0;
  const int m = live ? (int)(idx - blk * a.Mp) : 0;
  float v = 0.0f;
  if (live && m < a.M) {
    const int64_t s = a.src_off + blk * a.src_blk + (int64_t)m * D + d;
    v = a.src_bf16 ? (float)reinterpret_cast<const __bf16*>(a.src)[s] : reinterpret_cast<const float*>(a.src)[s];
  }
  float n2 = v * v;
#pragma unroll
  for (int off = D / 2; off >= 1; off >>= 1) n2 += __shfl_xor(n2, off);
  if (!live) return;
  if (a.op_hi) {
    const float xs = v * a.c;
    const __bf16 hi = (__bf16)xs;
    a.op_hi[idx * D + d] = hi;
    if (a.op_lo) a.op_lo[idx * D + d] = (__bf16)(xs - (float)hi);
  }
  if (a.op_zt) a.op_zt[(blk * D + d) * (int64_t)a.Mp + m] = (__bf16)v;
  if (a.qnorm && d == 0) a.qnorm[idx] = sqrtf(n2);
}

}  // namespace flarepp

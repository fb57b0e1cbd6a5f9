// Decode on bf16 matrix cores: every token reads the M latents back,
//     Y_n = sum_m softmax_m(s <K_n, Qd_m>) Z_m
// (FLARE summary, "Основной механизм FLARE", decode step Y = SDPA(K, Q, Z);
// the decode weights are row-softmaxed over the latents, section
// "Матрица коммуникации низкого ранга").
//
// Work decomposition.  A 256-thread workgroup owns one (b, h) and a chunk of
// tokens.  Every wave keeps the whole latent side in registers for its
// lifetime (c * Qd as a bf16 hi/lo pair, or for heads within the fp16 logit
// bound as one fp16 operand against keys converted to fp16 after each load
// (f16_logits, common.h), and Z^T, as matrix-core operands), and streams 16-token
// blocks of K straight from global memory (each lane 16 contiguous bytes of
// one token row), two blocks ahead of the one it consumes.
// Per block a wave computes L^T = Qd K^T (rows = latents, cols = tokens) for
// all M latents, so the softmax over M is a reduction over registers plus one
// pair of cross-row permlane swaps, then Y^T += Z^T P^T on the matrix cores
// (the weights feed the second product without leaving registers; see
// common.h), and writes Y rows as 16-byte stores (a wave writes 16 whole rows).
//
// Shift.  mu_n = |c| ||K_n|| max_m ||Qd_m|| bounds every logit of token n
// (Cauchy-Schwarz); when 2 mu_n <= 100 for all tokens of a block it enters as
// the MFMA accumulator input and no per-score max is taken.  Otherwise the
// block first takes the exact max over m in a logits-only pass.  Either way
// the weights are the softmax up to rounding; the sum uses the same
// bf16-rounded weights that enter Z^T P^T (a matrix-core product with a tile
// of ones).  Logits are produced and consumed
// four 16-latent blocks at a time so they stay in VGPRs.
#pragma once

#include "common.h"
#include "encode_bf16.h"
#include "merge.h"

namespace flarepp {

struct DecodeArgs {
  const __bf16* q_hi;   // Mp x D blocks of bf16(c * Qd)
  const __bf16* q_lo;   // Mp x D blocks of bf16(c * Qd - hi)
  int64_t q_sb, q_sh, q_off;  // (b, h)'s block starts at element b*q_sb + h*q_sh - q_off
  const float* qnorm;   // ||Qd_m|| with the same block layout divided by D, or null
  const float* knorm;   // [G][Jk] largest squared key norm of each split of the head (from the seed
                        // encode), or null
  int Jk;
  const __bf16* zt;     // [G][D][Mp] bf16(Z), transposed (G = heads of this launch)
  const __bf16* K;      // B x H x N x D
  float* Y;             // B x H x N x D
  int H, N, M, Mp, chunk;
  int64_t bh0;
  float c;
};

// One shift for every token of the head: mu_g = |c| max_n ||K_n|| max_m ||Qd_m||
// bounds every logit of the head (Cauchy-Schwarz, with a relative margin for
// the rounding of the hi/lo operand); when 2 mu_g <= kBoundSpan all logits lie
// in [-2 mu_g, 0] after the shift and no per-token norm is needed.  Needs the
// split key norms of the head (a.knorm) and the latent norms; +inf otherwise.
// kmax receives max_n ||K_n|| (+inf without the key norms).
__device__ __forceinline__ float head_shift(const DecodeArgs& a, int64_t lbh, float qmax, int lane, float& kmax) {
  kmax = INFINITY;
  if (!a.knorm || !a.qnorm) return INFINITY;
  float k2 = 0.0f;
  for (int j = lane; j < a.Jk; j += 64) k2 = fmaxf(k2, a.knorm[lbh * a.Jk + j]);
  kmax = __builtin_sqrtf(wave_max(k2));
  return fabsf(a.c) * kmax * qmax * (1.0f + 1.0f / 4096.0f);
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

template <int D, int MB>
__global__ __launch_bounds__(256, 1) void decode_bf16(DecodeArgs a) {
  constexpr int KL = KOperand<D>::kLen;
  constexpr int DB = D / 16;
  constexpr int KB = (MB + 1) / 2;     // 32-latent contraction blocks of Z^T P^T
  constexpr int MP = MB * 16;
  typedef typename KOperand<D>::T kop_t;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const int n0 = blockIdx.x * a.chunk;
  const int n1 = min(a.N, n0 + a.chunk);

  // ---- the whole latent side lives in registers for the workgroup's lifetime
  const int64_t qo = (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off;
  kop_t qh[MB], ql[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t o = qo + (int64_t)(mb * 16 + c16) * D + KL * g;
    qh[mb] = *reinterpret_cast<const kop_t*>(a.q_hi + o);
    ql[mb] = *reinterpret_cast<const kop_t*>(a.q_lo + o);
  }
  bf16x8 zop[KB][DB];
  {
    const __bf16* zb = a.zt + lbh * (int64_t)MP * D;
#pragma unroll
    for (int kb2 = 0; kb2 < KB; ++kb2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const __bf16* zr = zb + (int64_t)(16 * db + c16) * MP + kb2 * 32 + 4 * g;
        const bf16x4 z0 = *reinterpret_cast<const bf16x4*>(zr);
        bf16x4 z1 = bf16x4{};
        if (2 * kb2 + 1 < MB) z1 = *reinterpret_cast<const bf16x4*>(zr + 16);
        zop[kb2][db] = bf16x8{z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
      }
  }
  float qmax = 0.0f;
  if (a.qnorm)
    for (int m = lane; m < MP; m += 64) qmax = fmaxf(qmax, a.qnorm[qo / D + m]);
  qmax = wave_max(qmax);
  const bool have_bound = a.qnorm != nullptr;
  const bool ragged_m = a.M < MP;
  float kmax;
  const float mu_g = head_shift(a, lbh, qmax, lane, kmax);
  const bool gshift = 2.0f * mu_g <= kBoundSpan;
  const bool q16 = f16_logits(mu_g, kmax, qmax, a.c);

  // K and Y of this workgroup's tokens as buffer resources: tokens past n1
  // read as zeros and their stores are dropped, so loads need no clamping
  // and stay in flight across iterations
  const int nt = max(n1 - n0, 0);
  const __amdgpu_buffer_rsrc_t Kr = buffer_rsrc(a.K + (bh * (int64_t)a.N + n0) * D, (uint32_t)nt * D * 2);
  const __amdgpu_buffer_rsrc_t Yr = buffer_rsrc(a.Y + (bh * (int64_t)a.N + n0) * D, (uint32_t)nt * D * 4);
  const int kvoff = ((wave * 16 + c16) * D + KL * g) * 2;  // blk - n0 = wave * 16 + 64 j
  auto kload = [&](int blk) { return buffer_load<kop_t>(Kr, kvoff + (blk - n0 - wave * 16) * D * 2); };
  constexpr int CH = MB < 4 ? MB : 4;     // latent blocks per chunk of logits
  constexpr int NCH = (MB + CH - 1) / CH;

  // A operand of the weight-sum tile: all ones, so every row of ONES P^T is
  // the per-token sum of the same bf16 weights that enter Z^T P^T
  const bf16x8 ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                       (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
  // the token loop, compiled once with the hi/lo logits and once with the
  // fp16 ones (Q16); the head's bound picks one for the whole workgroup
  auto run = [&](auto q16_tag) {
  constexpr bool Q16 = decltype(q16_tag)::value;
  typedef typename KOperand16<D>::T hop_t;
  hop_t qf[Q16 ? MB : 1];
  if constexpr (Q16) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) qf[mb] = to_f16<hop_t>(qh[mb], ql[mb]);
  }
  auto body = [&](const kop_t kb, const int blk) {

    float sh = -mu_g;
    hop_t k16;
    if constexpr (Q16) k16 = to_f16<hop_t>(kb);
    if (!Q16 && !gshift) {  // (Q16 implies gshift)
      // token norm -> shift
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < KL / 2; ++e) {
        const bf16x2 pr = {kb[2 * e], kb[2 * e + 1]};
        ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
      }
      ss = sum_over_rows(ss);
      const float mu = fabsf(a.c) * __builtin_amdgcn_sqrtf(ss) * qmax * (1.0f + 1.0f / 4096.0f);
      const bool use_bound = have_bound && !__any(!(2.0f * mu <= kBoundSpan));
      sh = -mu;
      if (!use_bound) {
        // exact max over the latents: a logits-only pass
        float lm = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          f32x4 t = KOperand<D>::mma(qh[mb], kb, f32x4{0.f, 0.f, 0.f, 0.f});
          t = KOperand<D>::mma(ql[mb], kb, t);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (!ragged_m || mb < MB - 1 || (MB - 1) * 16 + 4 * g + r < a.M) lm = fmaxf(lm, t[r]);
        }
        sh = -max_over_rows(lm);
      }
    }
    const f32x4 cinit = {sh, sh, sh, sh};

    f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
    f32x4 yacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) yacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      f32x4 L[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int mb = ch * CH + i;
        if (mb < MB) {
          if constexpr (Q16) {
            L[i] = KOperand16<D>::mma(qf[mb], k16, cinit);
          } else {
            L[i] = KOperand<D>::mma(qh[mb], kb, cinit);
            L[i] = KOperand<D>::mma(ql[mb], kb, L[i]);
          }
        } else {
          L[i] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
      }
      if (ragged_m && ch == NCH - 1) {
#pragma unroll
        for (int i = 0; i < CH; ++i)
          if (ch * CH + i == MB - 1)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if ((MB - 1) * 16 + 4 * g + r >= a.M) L[i][r] = -INFINITY;
      }
#pragma unroll
      for (int i2 = 0; i2 < CH / 2 + (CH & 1); ++i2) {
        const int kb2 = ch * (CH / 2) + i2;  // CH is even whenever NCH > 1
        if (kb2 >= KB) break;
        const bf16x2 p0 = pack_bf16(fast_exp2(L[2 * i2][0]), fast_exp2(L[2 * i2][1]));
        const bf16x2 p1 = pack_bf16(fast_exp2(L[2 * i2][2]), fast_exp2(L[2 * i2][3]));
        bf16x2 p2 = {(__bf16)0.0f, (__bf16)0.0f}, p3 = p2;
        if (2 * i2 + 1 < CH) {
          p2 = pack_bf16(fast_exp2(L[2 * i2 + 1][0]), fast_exp2(L[2 * i2 + 1][1]));
          p3 = pack_bf16(fast_exp2(L[2 * i2 + 1][2]), fast_exp2(L[2 * i2 + 1][3]));
        }
        const bf16x8 pb = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
        for (int db = 0; db < DB; ++db) yacc[db] = mfma_k32(zop[kb2][db], pb, yacc[db]);
        lacc = mfma_k32(ones, pb, lacc);
      }
    }
    const float inv = __builtin_amdgcn_rcpf(lacc[0]);
    const int yoff = ((blk - n0 + c16) * D + 4 * g) * 4;
#pragma unroll
    for (int db = 0; db < DB; ++db) buffer_store(yacc[db] * inv, Yr, yoff + 64 * db);
  };

  // Two 16-token blocks of K in flight ahead of the one being consumed.  The
  // loop is unrolled by three so every block's registers are loaded once and
  // consumed in place (copying a register that a load is still filling would
  // make the copy wait for that load).
  // Whole groups of three blocks (blocks past the chunk read its last row and
  // store nothing), so the loop has a single steady state.
  constexpr int S = 64;
  int blk = n0 + wave * 16;
  // k0 is issued before k1 (kept in that order), so that the loop's first
  // wait for k0 leaves k1 in flight on the entry path as on the back edge
  kop_t k0 = kload(blk);
  __builtin_amdgcn_sched_barrier(0);
  kop_t k1 = kload(blk + S), k2;
  for (; blk < n1; blk += 3 * S) {
    k2 = kload(blk + 2 * S);
    body(k0, blk);
    k0 = kload(blk + 3 * S);
    body(k1, blk + S);
    k1 = kload(blk + 4 * S);
    body(k2, blk + 2 * S);
  }
  };
  if (q16)
    run(Flag<true>{});
  else
    run(Flag<false>{});
}

// Paired decode for many latents.  Holding c * Qd (hi/lo) and Z^T for all M
// latents costs one wave ~190 VGPRs at M = 256 (one wave per SIMD, nothing to
// hide the MFMA -> exp -> MFMA dependencies).  Here two waves share every
// 16-token block, each owning MBH of the latent blocks; both compute the
// same per-token shift, so their partial weight sums and partial Y^T tiles
// add exactly, and they swap the halves each one stores through a
// double-buffered LDS exchange (one barrier per block).  When a block needs
// the exact max over the latents (the bound is unsafe), the two partial
// maxima are exchanged the same way first.
constexpr uint32_t kWaitLgkm0 = 0xF | (0x7 << 4) | (0x3 << 14);  // s_waitcnt lgkmcnt(0)

__device__ __forceinline__ void pair_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// RAGGED: some of this wave's latent rows lie at or past M (M is not a
// multiple of 16, or the blocks do not split evenly); those get weight zero.
//
// Q16: the kernel serves the heads whose logits take one fp16 product
// (f16_logits) and returns at once for the others; the route launches both
// forms back to back.  The fp16 form holds one operand per latent block
// instead of the hi/lo pair and fits 128 VGPRs: four waves per SIMD.
template <int D, int MBH, bool RAGGED, bool Q16>
__global__ __launch_bounds__(128, Q16 ? 4 : 2) void decode_pair_bf16(DecodeArgs a) {
  constexpr int KL = KOperand<D>::kLen;
  constexpr int DB = D / 16;
  constexpr int KBH = (MBH + 1) / 2;  // 32-latent contraction blocks per wave
  typedef typename KOperand<D>::T kop_t;
  __shared__ f32x4 sY[2][2][64];      // [buffer][sender][lane]
  __shared__ float sLam[2][2][16];    // [buffer][sender][token]
  __shared__ float sMax[2][16];       // [sender][token]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w2 = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const int n0 = blockIdx.x * a.chunk;
  const int n1 = min(a.N, n0 + a.chunk);
  const int MB = a.Mp >> 4;
  const int mb0 = w2 * MBH;  // this wave's first latent block
  const int64_t qo = (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off;

  float qmax = 0.0f;
  if (a.qnorm)
    for (int m = lane; m < a.Mp; m += 64) qmax = fmaxf(qmax, a.qnorm[qo / D + m]);
  qmax = wave_max(qmax);
  const bool have_bound = a.qnorm != nullptr;
  float kmax;
  const float mu_g = head_shift(a, lbh, qmax, lane, kmax);
  const bool gshift = 2.0f * mu_g <= kBoundSpan;  // the same in both waves
  // the same in both waves, so the whole workgroup leaves together
  if (f16_logits(mu_g, kmax, qmax, a.c) != Q16) return;

  // ---- this wave's half of the latent side, in registers
  kop_t qh[MBH], ql[MBH];
#pragma unroll
  for (int i = 0; i < MBH; ++i) {
    if (mb0 + i < MB) {
      const int64_t o = qo + (int64_t)((mb0 + i) * 16 + c16) * D + KL * g;
      qh[i] = *reinterpret_cast<const kop_t*>(a.q_hi + o);
      ql[i] = *reinterpret_cast<const kop_t*>(a.q_lo + o);
    } else {
      qh[i] = kop_t{};
      ql[i] = kop_t{};
    }
  }
  bf16x8 zop[KBH][DB];
  {
    const __bf16* zb = a.zt + lbh * (int64_t)a.Mp * D;
#pragma unroll
    for (int kb = 0; kb < KBH; ++kb)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const __bf16* zr = zb + (int64_t)(16 * db + c16) * a.Mp + (mb0 + 2 * kb) * 16 + 4 * g;
        bf16x4 z0 = bf16x4{}, z1 = bf16x4{};
        if (mb0 + 2 * kb < MB) z0 = *reinterpret_cast<const bf16x4*>(zr);
        if (2 * kb + 1 < MBH && mb0 + 2 * kb + 1 < MB) z1 = *reinterpret_cast<const bf16x4*>(zr + 16);
        zop[kb][db] = bf16x8{z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
      }
  }
  // latent rows of this wave at or past M (the padding of the last block and
  // whole blocks past the end) get weight zero
  const int mvalid = a.M - mb0 * 16;
  // ragged: block ipart holds the first row at or past M (rows 4 g + r of it
  // with 4 g + r >= rem take padb = -inf); later blocks are all padding.
  // Additive per-lane biases keep the masks out of scalar registers.
  const int ipart = mvalid >> 4, rem = mvalid & 15;
  f32x4 padb;
#pragma unroll
  for (int r = 0; r < 4; ++r) padb[r] = 4 * g + r < rem ? 0.0f : -INFINITY;

  // K and Y of this workgroup's tokens as buffer resources: tokens past n1
  // read as zeros and their stores are dropped
  const int nt = max(n1 - n0, 0);
  const __amdgpu_buffer_rsrc_t Kr = buffer_rsrc(a.K + (bh * (int64_t)a.N + n0) * D, (uint32_t)nt * D * 2);
  const __amdgpu_buffer_rsrc_t Yr = buffer_rsrc(a.Y + (bh * (int64_t)a.N + n0) * D, (uint32_t)nt * D * 4);
  const int kvoff = (c16 * D + KL * g) * 2;
  auto kload = [&](int blk) { return buffer_load<kop_t>(Kr, kvoff + (blk - n0) * D * 2); };

  // A operand of the weight-sum tile: all ones, so every row of ONES P^T is
  // the per-token sum of the same bf16 weights that enter Z^T P^T
  const bf16x8 ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                       (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
  auto run = [&](auto q16_tag) {
  static_assert(decltype(q16_tag)::value == Q16, "one logit form per kernel");
  typedef typename KOperand16<D>::T hop_t;
  hop_t qf[Q16 ? MBH : 1];
  if constexpr (Q16) {
#pragma unroll
    for (int i = 0; i < MBH; ++i) qf[i] = to_f16<hop_t>(qh[i], ql[i]);
  }
  auto body = [&](const kop_t kb, const int blk, const int buf) {

    float sh = -mu_g;
    hop_t k16;
    if constexpr (Q16) k16 = to_f16<hop_t>(kb);
    if (!Q16 && !gshift) {  // (Q16 implies gshift)
      // token norm -> shift (identical in both waves)
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < KL / 2; ++e) {
        const bf16x2 pr = {kb[2 * e], kb[2 * e + 1]};
        ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
      }
      ss = sum_over_rows(ss);
      const float mu = fabsf(a.c) * __builtin_amdgcn_sqrtf(ss) * qmax * (1.0f + 1.0f / 4096.0f);
      const bool use_bound = have_bound && __builtin_amdgcn_ballot_w64(!(2.0f * mu <= kBoundSpan)) == 0;
      sh = -mu;
      if (!use_bound) {
        // exact max over all latents: this wave's half, then the partner's
        float lm = -INFINITY;
#pragma unroll
        for (int i = 0; i < MBH; ++i) {
          if (RAGGED && i > ipart) continue;
          f32x4 t = KOperand<D>::mma(qh[i], kb, f32x4{0.f, 0.f, 0.f, 0.f});
          t = KOperand<D>::mma(ql[i], kb, t);
          if (RAGGED && i == ipart) t += padb;
#pragma unroll
          for (int r = 0; r < 4; ++r) lm = fmaxf(lm, t[r]);
        }
        lm = max_over_rows(lm);
        if (g == 0) sMax[w2][c16] = lm;
        pair_barrier();
        sh = -fmaxf(lm, sMax[1 - w2][c16]);
        pair_barrier();  // both have read sMax before it is written again
      }
    }
    const f32x4 cinit = {sh, sh, sh, sh};

    f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
    f32x4 yacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) yacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb2 = 0; kb2 < KBH; ++kb2) {
      f32x4 L[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = 2 * kb2 + u;
        if (i < MBH) {
          if constexpr (Q16) {
            L[u] = KOperand16<D>::mma(qf[i], k16, cinit);
          } else {
            L[u] = KOperand<D>::mma(qh[i], kb, cinit);
            L[u] = KOperand<D>::mma(ql[i], kb, L[u]);
          }
          if (RAGGED) {
            if (i == ipart)
              L[u] += padb;
            else if (i > ipart)
              L[u] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
          }
        } else {
          L[u] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
      }
      const bf16x2 p0 = pack_bf16(fast_exp2(L[0][0]), fast_exp2(L[0][1]));
      const bf16x2 p1 = pack_bf16(fast_exp2(L[0][2]), fast_exp2(L[0][3]));
      const bf16x2 p2 = pack_bf16(fast_exp2(L[1][0]), fast_exp2(L[1][1]));
      const bf16x2 p3 = pack_bf16(fast_exp2(L[1][2]), fast_exp2(L[1][3]));
      const bf16x8 pb = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
      for (int db = 0; db < DB; ++db) yacc[db] = mfma_k32(zop[kb2][db], pb, yacc[db]);
      lacc = mfma_k32(ones, pb, lacc);
    }
    const float lam = lacc[0];

    // swap: wave w2 stores d-block w2 (D = 32) or wave 0 stores all (D = 16)
    if (g == 0) sLam[buf][w2][c16] = lam;
    const int yoff = ((blk - n0 + c16) * D + 4 * g) * 4;
    if (w2 == 0) {
      if (DB == 2) sY[buf][0][lane] = yacc[DB - 1];
      pair_barrier();
      const float inv = __builtin_amdgcn_rcpf(lam + sLam[buf][1][c16]);
      const f32x4 y = yacc[0] + sY[buf][1][lane];
      buffer_store(y * inv, Yr, yoff);
    } else {
      sY[buf][1][lane] = yacc[0];
      pair_barrier();
      if (DB == 2) {
        const float inv = __builtin_amdgcn_rcpf(lam + sLam[buf][0][c16]);
        const f32x4 y = yacc[DB - 1] + sY[buf][0][lane];
        buffer_store(y * inv, Yr, yoff + 64);
      }
    }
  };

  // two blocks in flight ahead; unrolled by three (see decode_bf16), and by
  // two more for the exchange buffer's parity
  constexpr int S = 16;
  int blk = n0;
  // k0 is issued before k1 (kept in that order), so that the loop's first
  // wait for k0 leaves k1 in flight on the entry path as on the back edge
  kop_t k0 = kload(blk);
  __builtin_amdgcn_sched_barrier(0);
  kop_t k1 = kload(blk + S), k2;
  for (int it = 0; blk < n1; blk += 3 * S, ++it) {
    const int par = it & 1;  // blocks 3 it .. 3 it + 2 use buffers par, !par, par
    k2 = kload(blk + 2 * S);
    body(k0, blk, par);
    k0 = kload(blk + 3 * S);
    body(k1, blk + S, par ^ 1);
    k1 = kload(blk + 4 * S);
    body(k2, blk + 2 * S, par);
  }
  };
  run(Flag<Q16>{});
}

}  // namespace flarepp

// Decode on bf16 matrix cores: every token reads the M latents back,
//     Y_n = sum_m softmax_m(s <K_n, Qd_m>) Z_m
// (FLARE summary, "Основной механизм FLARE", decode step Y = SDPA(K, Q, Z);
// the decode weights are row-softmaxed over the latents, section
// "Матрица коммуникации низкого ранга").
//
// Work decomposition.  A 256-thread workgroup owns one (b, h) and a chunk of
// tokens.  Every wave keeps the whole latent side in registers for its
// lifetime (c * Qd as a bf16 hi/lo pair and Z^T, as matrix-core operands:
// ~200 VGPRs at M = 256, D = 32, one wave per SIMD), and streams 16-token
// blocks of K straight from global memory (each lane 16 contiguous bytes of
// one token row), two blocks ahead of the one it consumes.
// Per block a wave computes L^T = Qd K^T (rows = latents, cols = tokens) for
// all M latents, so the softmax over M is a reduction over registers plus one
// pair of cross-row permlane swaps, then Y^T += Z^T P^T on the matrix cores
// (the weights feed the second product without leaving registers; see
// common.h), and writes Y rows as 16-byte stores (a wave writes 16 whole rows).
//
// Shift.  mu_n = c ||K_n|| max_m ||Qd_m|| bounds every logit of token n
// (Cauchy-Schwarz); when 2 mu_n <= 100 for all tokens of a block it enters as
// the MFMA accumulator input and no per-score max is taken.  Otherwise the
// block first takes the exact max over m in a logits-only pass.  Either way
// the weights are the softmax up to rounding; the sum uses the same
// bf16-rounded weights that enter Z^T P^T.  Logits are produced and consumed
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
  const __bf16* zt;     // [G][D][Mp] bf16(Z), transposed (G = heads of this launch)
  const __bf16* K;      // B x H x N x D
  float* Y;             // B x H x N x D
  int H, N, M, Mp, chunk;
  int64_t bh0;
  float c;
};

template <int D, int MB>
__global__ __launch_bounds__(256, 1) void decode_bf16(DecodeArgs a) {
  constexpr int KL = KOperand<D>::kLen;
  constexpr int DB = D / 16;
  constexpr int KB = (MB + 1) / 2;     // 32-latent contraction blocks of Z^T P^T
  constexpr int MP = MB * 16;
  typedef typename KOperand<D>::T kop_t;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  const __bf16* Kp = a.K + bh * (int64_t)a.N * D;
  float* Yp = a.Y + bh * (int64_t)a.N * D;
  // Branch-free loads: a token past the chunk reads the chunk's last row
  // (its results are never stored), so loads can stay in flight across
  // iterations.
  auto kload = [&](int blk) {
    const int tok = min(blk + c16, n1 - 1);
    return *reinterpret_cast<const kop_t*>(Kp + (int64_t)tok * D + KL * g);
  };
  constexpr int CH = MB < 4 ? MB : 4;     // latent blocks per chunk of logits
  constexpr int NCH = (MB + CH - 1) / CH;

  // two 16-token blocks of K in flight ahead of the one being consumed
  int blk = n0 + wave * 16;
  kop_t k1 = kload(blk), k2 = kload(blk + 64);
  for (; blk < n1; blk += 64) {
    const kop_t kb = k1;
    k1 = k2;
    k2 = kload(blk + 128);
    const int tok = blk + c16;

    // token norm -> shift
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < KL / 2; ++e) {
      const bf16x2 pr = {kb[2 * e], kb[2 * e + 1]};
      ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
    }
    ss = sum_over_rows(ss);
    const float mu = a.c * sqrtf(ss) * qmax * (1.0f + 1.0f / 4096.0f);
    const bool use_bound = have_bound && !__any(!(2.0f * mu <= kBoundSpan));
    float sh = -mu;
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
    const f32x4 cinit = {sh, sh, sh, sh};

    float lam = 0.0f;
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
          L[i] = KOperand<D>::mma(qh[mb], kb, cinit);
          L[i] = KOperand<D>::mma(ql[mb], kb, L[i]);
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
        lam = add_pair(p3, add_pair(p2, add_pair(p1, add_pair(p0, lam))));
        const bf16x8 pb = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
        for (int db = 0; db < DB; ++db) yacc[db] = mfma_k32(zop[kb2][db], pb, yacc[db]);
      }
    }
    const float inv = 1.0f / sum_over_rows(lam);
    if (tok < n1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(Yp + (int64_t)tok * D + 16 * db + 4 * g) = yacc[db] * inv;
    }
  }
}

}  // namespace flarepp

// Decode on bf16 matrix cores: every token reads the M latents back,
//     Y_n = sum_m softmax_m(s <K_n, Qd_m>) Z_m
// (FLARE summary, "Основной механизм FLARE", decode step Y = SDPA(K, Q, Z);
// the decode weights are row-softmaxed over the latents, section
// "Матрица коммуникации низкого ранга").
//
// Work decomposition.  A 256-thread workgroup owns one (b, h) and a chunk of
// tokens; it stages the whole Qd operand (c * Qd as bf16 hi/lo) and Z^T in
// LDS once, then each wave streams 16-token blocks of K straight from global
// memory into registers (each lane 16 contiguous bytes of one token row).
// Per block a wave computes L^T = Qd K^T (rows = latents, cols = tokens) for
// all M latents, so the softmax over M is a reduction over registers plus one
// pair of cross-row permlane swaps, then Y^T += Z^T P^T on the matrix cores
// (the weights feed the second product without leaving registers; see
// common.h), and writes Y rows as 16-byte stores (a wave writes 16 whole rows).
//
// Shift.  mu_n = c ||K_n|| max_m ||Qd_m|| bounds every logit of token n
// (Cauchy-Schwarz); when 2 mu_n <= 100 for all tokens of a block it enters as
// the MFMA accumulator input and no per-score max is taken.  Otherwise the
// block takes the exact max over m.  Either way the weights are the softmax up
// to rounding; the sum uses the same bf16-rounded weights that enter Z^T P^T.
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
  constexpr int ZROW = KB * 32 + 8;    // transposed-Z row stride (elements)
  typedef typename KOperand<D>::T kop_t;

  __shared__ __attribute__((aligned(16))) __bf16 sQh[MP * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQl[MP * D];
  __shared__ __attribute__((aligned(16))) __bf16 sZt[D * ZROW];
  __shared__ float sQmax[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int n0 = blockIdx.x * a.chunk;
  const int n1 = min(a.N, n0 + a.chunk);

  // ---- stage Qd (hi, lo) and Z^T for this (b, h) in LDS
  {
    const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
    const int64_t qo = (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off;
    for (int u = tid; u < MP * D / 8; u += 256) {
      *reinterpret_cast<uint4*>(&sQh[u * 8]) = *reinterpret_cast<const uint4*>(a.q_hi + qo + u * 8);
      *reinterpret_cast<uint4*>(&sQl[u * 8]) = *reinterpret_cast<const uint4*>(a.q_lo + qo + u * 8);
    }
    const int64_t ob = lbh * (int64_t)MP * D;
    for (int u = tid; u < D * (ZROW / 8); u += 256) {
      const int d = u / (ZROW / 8), m8 = (u % (ZROW / 8)) * 8;
      *reinterpret_cast<uint4*>(&sZt[d * ZROW + m8]) =
          (m8 < MP) ? *reinterpret_cast<const uint4*>(a.zt + ob + (int64_t)d * MP + m8) : make_uint4(0, 0, 0, 0);
    }
    float qm = 0.0f;
    if (a.qnorm)
      for (int m = tid; m < MP; m += 256) qm = fmaxf(qm, a.qnorm[qo / D + m]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) qm = fmaxf(qm, __shfl_xor(qm, off));
    if (lane == 0) sQmax[wave] = qm;
  }
  __syncthreads();
  const float qmax = fmaxf(fmaxf(sQmax[0], sQmax[1]), fmaxf(sQmax[2], sQmax[3]));
  const bool have_bound = a.qnorm != nullptr;
  const bool ragged_m = a.M < MP;

  const __bf16* Kp = a.K + bh * (int64_t)a.N * D;
  float* Yp = a.Y + bh * (int64_t)a.N * D;

  for (int blk = n0 + wave * 16; blk < n1; blk += 64) {
    const int tok = blk + c16;
    const bool tok_ok = tok < n1;
    const kop_t kb = tok_ok ? *reinterpret_cast<const kop_t*>(Kp + (int64_t)tok * D + KL * g) : kop_t{};

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
    const float sh = use_bound ? -mu : 0.0f;
    const f32x4 cinit = {sh, sh, sh, sh};

    f32x4 L[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const kop_t qh = *reinterpret_cast<const kop_t*>(&sQh[(mb * 16 + c16) * D + KL * g]);
      const kop_t ql = *reinterpret_cast<const kop_t*>(&sQl[(mb * 16 + c16) * D + KL * g]);
      L[mb] = KOperand<D>::mma(qh, kb, cinit);
      L[mb] = KOperand<D>::mma(ql, kb, L[mb]);
    }
    if (ragged_m) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if ((MB - 1) * 16 + 4 * g + r >= a.M) L[MB - 1][r] = -INFINITY;
    }
    if (!use_bound) {
      float lm = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) lm = fmaxf(lm, fmaxf(max3(L[mb][0], L[mb][1], L[mb][2]), L[mb][3]));
      lm = max_over_rows(lm);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) L[mb] -= lm;
    }

    float lam = 0.0f;
    f32x4 yacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) yacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb2 = 0; kb2 < KB; ++kb2) {
      const bf16x2 p0 = pack_bf16(fast_exp2(L[2 * kb2][0]), fast_exp2(L[2 * kb2][1]));
      const bf16x2 p1 = pack_bf16(fast_exp2(L[2 * kb2][2]), fast_exp2(L[2 * kb2][3]));
      bf16x2 p2 = {(__bf16)0.0f, (__bf16)0.0f}, p3 = p2;
      if (2 * kb2 + 1 < MB) {
        p2 = pack_bf16(fast_exp2(L[2 * kb2 + 1][0]), fast_exp2(L[2 * kb2 + 1][1]));
        p3 = pack_bf16(fast_exp2(L[2 * kb2 + 1][2]), fast_exp2(L[2 * kb2 + 1][3]));
      }
      lam = add_pair(p3, add_pair(p2, add_pair(p1, add_pair(p0, lam))));
      const bf16x8 pb = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const __bf16* zr = &sZt[(16 * db + c16) * ZROW + kb2 * 32 + 4 * g];
        const bf16x4 z0 = *reinterpret_cast<const bf16x4*>(zr);
        const bf16x4 z1 = *reinterpret_cast<const bf16x4*>(zr + 16);
        const bf16x8 zop = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
        yacc[db] = mfma_k32(zop, pb, yacc[db]);
      }
    }
    const float inv = 1.0f / sum_over_rows(lam);
    if (tok_ok) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(Yp + (int64_t)tok * D + 16 * db + 4 * g) = yacc[db] * inv;
    }
  }
}

}  // namespace flarepp

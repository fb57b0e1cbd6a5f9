// Backward of the route for bf16 inputs on the matrix cores: the gradients
// dS, dK, dV (float32) of a scalar loss given dY (float32).  The chain rule
// is the one of the float32 path (backward_f32.h): for an SDPA application
// O = SDPA(Q, K, V, s) with P_ij = softmax_j(s <Q_i, K_j>) and upstream dO,
//     dV_j += sum_i P_ij dO_i,   dL_ij = P_ij (<dO_i, V_j> - <dO_i, O_i>),
//     dQ_i += s sum_j dL_ij K_j, dK_j  += s sum_i dL_ij Q_i,
// taken through the decode (queries = tokens, keys = Qd, values = Z), the
// encode and the seed encode (FLARE summary, "Основной механизм FLARE").
//
// Each stage has a token pass (a workgroup owns tokens and walks all
// latents, whose operands it stages in LDS once) and a latent pass (a
// workgroup owns one split of the tokens and all latents, wave w latents
// 32 w .. 32 w + 31, and writes split partials that bwd_reduce sums).  Every
// contraction is a 16x16 MFMA tile with float32 accumulation:
//   * logits t = c <q, k> (log2 units, c = s log2 e) take the query as a
//     bf16 hi/lo pair (K is exact in bf16), so their error is that of
//     float32 arithmetic;
//   * <dO, V> takes dO as a bf16 hi/lo pair (V exact): the difference
//     <dO_i, V_j> - <dO_i, O_i> = <dO_i, V_j - O_i> is small for the tokens
//     that dominate a sharp softmax, so both terms need float32 accuracy;
//   * the decode's <dY_n, Z_m> - <dY_n, Y_n> is a difference of two averages
//     of the values when the softmax is broad, so it is formed as
//     <dY_n, Z'_m> - <dY_n, Y'_n> with Z' = Z - mean_m Z (the same number:
//     the weights of a token sum to one), Z' and dY as bf16 hi/lo pairs
//     (three products: hi hi, lo hi, hi lo);
//   * the products that form gradients (P dO, dL Q, P dY, dL K) take bf16
//     weights and bf16 operands: 2^-9 relative rounding per term.
// The C tile of a logit product leaves each lane one column and four rows;
// two such tiles are the eight k slots of the next product's operand in
// registers (common.h).  Transposed operands are read from LDS copies laid
// out [d][m] (latents) or [d][token].
#pragma once

#include "common.h"
#include "encode_bf16.h"

namespace flarepp {

constexpr int kBwdBf16MaxM = 256;
// LDS row stride (elements) of a transposed latent operand [D][m]: a read
// of 8 bytes by lane (row d = l mod 16, column 32 kb + 4 g) then starts 4
// banks apart per row and 2 per g, two wave passes as for a contiguous read.
constexpr int kBwdTS = kBwdBf16MaxM + 8;
// LDS row stride (elements) of a transposed 32-token tile [D][token]
constexpr int kBwdTT = 32 + 8;

// Latent-side operands of a stage as bf16 from float32 (or bf16) rows.
// Block k of the source is its rows src + k * src_blk ([M][D]); output
// block k: row-major hi/lo of alpha * x in [Mp][D] (rows M .. Mp - 1 zero),
// transposed x in [D][Mt] (columns M .. Mt - 1 zero); x = row - mean row
// when center is set.
struct BwdPrepArgs {
  const void* src;
  int src_bf16;
  int64_t src_blk;
  int M, Mp, Mt;
  int center;
  float alpha;
  __bf16* hi;  // or null
  __bf16* lo;  // or null
  __bf16* tr;  // or null
};

template <int D>
__global__ __launch_bounds__(256) void bwd_prep_bf16(BwdPrepArgs a) {
  __shared__ float smean[D];
  const int k = blockIdx.x, tid = threadIdx.x;
  auto load = [&](int m, int d) -> float {
    const int64_t i = (int64_t)k * a.src_blk + (int64_t)m * D + d;
    return a.src_bf16 ? (float)static_cast<const __bf16*>(a.src)[i] : static_cast<const float*>(a.src)[i];
  };
  if (a.center) {
    if (tid < D) {
      float s = 0.0f;
      for (int m = 0; m < a.M; ++m) s += load(m, tid);
      smean[tid] = s / (float)a.M;
    }
    __syncthreads();
  }
  for (int e = tid; e < a.Mt * D; e += 256) {
    const int m = e / D, d = e - m * D;
    const float x = m < a.M ? load(m, d) - (a.center ? smean[d] : 0.0f) : 0.0f;
    if (m < a.Mp && a.hi) {
      const float xs = a.alpha * x;
      const __bf16 h = (__bf16)xs;
      a.hi[(int64_t)k * a.Mp * D + e] = h;
      if (a.lo) a.lo[(int64_t)k * a.Mp * D + e] = (__bf16)(xs - (float)h);
    }
    if (a.tr) a.tr[((int64_t)k * D + d) * a.Mt + m] = (__bf16)x;
  }
}

// Arguments of the encode-stage passes (stages 1 and 2): queries Q
// (c Q as bf16 hi/lo rows and Q^T; (b, h)'s block at b * sb + h * sh - off,
// which also covers the seed blocks of stage 1), dO (bf16 rows and dO^T),
// the forward's per-latent log-sum-exp A_m and delta_m = <dO_m, O_m>.
struct BwdEncArgs {
  const __bf16* qhi;
  const __bf16* qlo;
  int64_t q_sb, q_sh, q_off;  // in [.][Mp][D] blocks
  const __bf16* qt;
  int64_t t_sb, t_sh, t_off;  // in [.][D][Mt] blocks
  const __bf16* dor;          // [G][Mp][D] dO as bf16 hi
  const __bf16* dorl;         // [G][Mp][D] bf16 lo (dO - hi)
  const __bf16* dot;          // [G][D][Mt]
  const float* lse;           // [G][Mp]
  const float* delta;         // [G][Mp]
  const __bf16* K;            // B x H x N x D
  const __bf16* V;
  float* dK;                  // token pass: B x H x N x D
  float* dV;
  int acc_dk, acc_dv;         // add into dK / dV (else overwrite)
  float* part;                // latent pass: [G][Mp][J][D]
  int J, chunk;               // latent pass: token splits
  int tchunk;                 // token pass: tokens per workgroup (multiple of 256)
  int H, N, M, Mp, Mt;
  int64_t bh0;
  float s;
};

// the bf16x8 operand of 32 latents (or tokens) kb: k slots 4 g .. 4 g + 3 and
// 16 + 4 g .. 16 + 4 g + 3 of LDS row `row`
__device__ __forceinline__ bf16x8 tr_operand(const __bf16* row, int c0, int g) {
  const bf16x4 x0 = *reinterpret_cast<const bf16x4*>(row + c0 + 4 * g);
  const bf16x4 x1 = *reinterpret_cast<const bf16x4*>(row + c0 + 16 + 4 * g);
  return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}

// weights of two C tiles (rows 4 g .. 4 g + 3 of tiles 0 and 1) as the k slots
// of one operand
__device__ __forceinline__ bf16x8 pack_tiles(f32x4 x0, f32x4 x1) {
  const bf16x2 p0 = pack_bf16(x0[0], x0[1]), p1 = pack_bf16(x0[2], x0[3]);
  const bf16x2 p2 = pack_bf16(x1[0], x1[1]), p3 = pack_bf16(x1[2], x1[3]);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ f32x4 splat4(float x) { return f32x4{x, x, x, x}; }

// Row-major [Mp][D] bf16 block -> LDS rows 0 .. Mt - 1 (zero past Mp).
template <int D>
__device__ __forceinline__ void stage_rows(__bf16* dst, const __bf16* src, int Mp, int Mt, int tid, int nthr) {
  for (int e = tid; e < Mt * D / 8; e += nthr) {
    bf16x8 v = bf16x8{};
    if (e < Mp * D / 8) v = reinterpret_cast<const bf16x8*>(src)[e];
    reinterpret_cast<bf16x8*>(dst)[e] = v;
  }
}
// Transposed [D][Mt] bf16 block -> LDS [D][kBwdTS].
template <int D>
__device__ __forceinline__ void stage_tr(__bf16* dst, const __bf16* src, int Mt, int tid, int nthr) {
  const int per = Mt / 8;
  for (int e = tid; e < D * per; e += nthr) {
    const int d = e / per, c = e - d * per;
    *reinterpret_cast<bf16x8*>(dst + d * kBwdTS + 8 * c) =
        *reinterpret_cast<const bf16x8*>(src + (int64_t)d * Mt + 8 * c);
  }
}

// K rows of 16 tokens as the B operand of a logit tile (lane: token
// n + l16, elements KL g ..), from a resource based at token n (tokens past
// the resource read as zeros).
template <int D>
__device__ __forceinline__ typename KOperand<D>::T tok_operand(const __bf16* base, int64_t n, int64_t nend,
                                                               int l16, int g) {
  constexpr int KL = KOperand<D>::kLen;
  const int64_t cnt = nend > n ? nend - n : 0;
  const __amdgpu_buffer_rsrc_t r = buffer_rsrc(base + n * D, (uint32_t)(cnt * D * 2));
  return buffer_load<typename KOperand<D>::T>(r, (l16 * D + KL * g) * 2);
}
// bf16 hi/lo pair of KL float32 elements (x0, then x1 when KL = 8)
template <int D>
__device__ __forceinline__ void split_hilo(f32x4 x0, f32x4 x1, typename KOperand<D>::T& hi,
                                           typename KOperand<D>::T& lo) {
  f32x4 r0, r1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r0[e] = x0[e] - (float)(__bf16)x0[e];
    r1[e] = x1[e] - (float)(__bf16)x1[e];
  }
  if constexpr (KOperand<D>::kLen == 8) {
    hi = pack_tiles(x0, x1);
    lo = pack_tiles(r0, r1);
  } else {
    const bf16x2 p0 = pack_bf16(x0[0], x0[1]), p1 = pack_bf16(x0[2], x0[3]);
    const bf16x2 q0 = pack_bf16(r0[0], r0[1]), q1 = pack_bf16(r0[2], r0[3]);
    hi = bf16x4{p0[0], p0[1], p1[0], p1[1]};
    lo = bf16x4{q0[0], q0[1], q1[0], q1[1]};
  }
}

// Raw float32 dY of 16 tokens from token n: the KL elements of the lane's
// operand slots (x0, x1) and, for the C-tile layout, elements 16 db + 4 g ..
// (y[db]).  Tokens past nend read as zeros.
template <int D>
struct DyRaw {
  f32x4 x0, x1, y[D / 16];
  __device__ __forceinline__ void load(const float* base, int64_t n, int64_t nend, int l16, int g) {
    constexpr int KL = KOperand<D>::kLen;
    const int64_t cnt = nend > n ? nend - n : 0;
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(base + n * D, (uint32_t)(cnt * D * 4));
    const int off = (l16 * D + KL * g) * 4;
    x0 = buffer_load<f32x4>(r, off);
    x1 = KL == 8 ? buffer_load<f32x4>(r, off + 16) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (D == 16) {
      y[0] = x0;  // elements 4 g .. 4 g + 3 either way
    } else {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) y[db] = buffer_load<f32x4>(r, (l16 * D + 16 * db + 4 * g) * 4);
    }
  }
};

// ---- encode-stage token pass: dV_n and dK_n of the workgroup's tokens.
// Wave w takes 32-token blocks tb = n0 + 32 w + 256 i; per 32-latent block
// kb: L = (c Q) K^T - A (rows latents, cols tokens), dP = dO V^T - delta,
// P = 2^L, dL = P dP, then dV^T += dO^T P and dK^T += Q^T dL.
template <int D>
__global__ __launch_bounds__(512) void bwd_enc_tok_bf16(BwdEncArgs a) {
  constexpr int KL = KOperand<D>::kLen;
  constexpr int DB = D / 16;
  typedef typename KOperand<D>::T kop_t;
  __shared__ __attribute__((aligned(16))) __bf16 sQh[kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQl[kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sDo[kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sDol[kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQt[D * kBwdTS];
  __shared__ __attribute__((aligned(16))) __bf16 sDot[D * kBwdTS];
  __shared__ __attribute__((aligned(16))) float sNA[kBwdBf16MaxM];
  __shared__ __attribute__((aligned(16))) float sND[kBwdBf16MaxM];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const int Mt = a.Mt, nkb = Mt / 32;
  stage_rows<D>(sQh, a.qhi + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off, a.Mp, Mt, tid, 512);
  stage_rows<D>(sQl, a.qlo + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off, a.Mp, Mt, tid, 512);
  stage_rows<D>(sDo, a.dor + lbh * a.Mp * D, a.Mp, Mt, tid, 512);
  stage_rows<D>(sDol, a.dorl + lbh * a.Mp * D, a.Mp, Mt, tid, 512);
  stage_tr<D>(sQt, a.qt + (int64_t)b * a.t_sb + (int64_t)h * a.t_sh - a.t_off, Mt, tid, 512);
  stage_tr<D>(sDot, a.dot + lbh * (int64_t)D * Mt, Mt, tid, 512);
  for (int m = tid; m < Mt; m += 512) {
    const bool real = m < a.M;
    sNA[m] = real ? -a.lse[lbh * a.Mp + m] : -INFINITY;
    sND[m] = real ? -a.delta[lbh * a.Mp + m] : 0.0f;
  }
  __syncthreads();

  const int64_t n0 = (int64_t)blockIdx.x * a.tchunk, n1 = min((int64_t)a.N, n0 + a.tchunk);
  const __bf16* Kh = a.K + bh * (int64_t)a.N * D;
  const __bf16* Vh = a.V + bh * (int64_t)a.N * D;
  // K and V of the next 32-token block are loaded while this one computes
  kop_t kn[2], vn[2];
  auto load_kv = [&](int64_t tb) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      kn[u] = tok_operand<D>(Kh, tb + 16 * u, n1, l16, g);
      vn[u] = tok_operand<D>(Vh, tb + 16 * u, n1, l16, g);
    }
  };
  if (n0 + 32 * w < n1) load_kv(n0 + 32 * w);
  for (int64_t tb = n0 + 32 * w; tb < n1; tb += 256) {
    kop_t kb_op[2], vb_op[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      kb_op[u] = kn[u];
      vb_op[u] = vn[u];
    }
    if (tb + 256 < n1) load_kv(tb + 256);
    f32x4 dvt[2][DB], dkt[2][DB];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) dvt[u][db] = dkt[u][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int kb = 0; kb < nkb; ++kb) {
      f32x4 P[2][2], dL[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int m0 = 32 * kb + 16 * t;
        const kop_t qh = *reinterpret_cast<const kop_t*>(sQh + (m0 + l16) * D + KL * g);
        const kop_t ql = *reinterpret_cast<const kop_t*>(sQl + (m0 + l16) * D + KL * g);
        const kop_t dov = *reinterpret_cast<const kop_t*>(sDo + (m0 + l16) * D + KL * g);
        const kop_t dol = *reinterpret_cast<const kop_t*>(sDol + (m0 + l16) * D + KL * g);
        const f32x4 na = *reinterpret_cast<const f32x4*>(sNA + m0 + 4 * g);
        const f32x4 nd = *reinterpret_cast<const f32x4*>(sND + m0 + 4 * g);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          f32x4 L = KOperand<D>::mma(qh, kb_op[u], na);
          L = KOperand<D>::mma(ql, kb_op[u], L);
          f32x4 dp = KOperand<D>::mma(dov, vb_op[u], nd);
          dp = KOperand<D>::mma(dol, vb_op[u], dp);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            P[t][u][r] = fast_exp2(L[r]);
            dL[t][u][r] = P[t][u][r] * dp[r];
          }
        }
      }
      bf16x8 pb[2], lb[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        pb[u] = pack_tiles(P[0][u], P[1][u]);
        lb[u] = pack_tiles(dL[0][u], dL[1][u]);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 dot = tr_operand(sDot + (16 * db + l16) * kBwdTS, 32 * kb, g);
        const bf16x8 qt = tr_operand(sQt + (16 * db + l16) * kBwdTS, 32 * kb, g);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          dvt[u][db] = mfma_k32(dot, pb[u], dvt[u][db]);
          dkt[u][db] = mfma_k32(qt, lb[u], dkt[u][db]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t n = tb + 16 * u + l16;
      if (n < n1) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int64_t o = (bh * (int64_t)a.N + n) * D + 16 * db + 4 * g;
          f32x4 kv = dkt[u][db] * a.s, vv = dvt[u][db];
          if (a.acc_dk) kv += *reinterpret_cast<const f32x4*>(a.dK + o);
          if (a.acc_dv) vv += *reinterpret_cast<const f32x4*>(a.dV + o);
          *reinterpret_cast<f32x4*>(a.dK + o) = kv;
          *reinterpret_cast<f32x4*>(a.dV + o) = vv;
        }
      }
    }
  }
}

// ---- encode-stage latent pass: split partials of dQ_m = s sum_n dL_mn K_n.
// Per 32-token step: L^T = K (c Q)^T - A (rows tokens, cols latents),
// dP^T = V dO^T - delta, dL = 2^L dP (zero past the split), dQ^T += K^T dL^T
// with K^T read from a transposed LDS copy of the step's tile.
template <int D>
__global__ __launch_bounds__(512) void bwd_enc_lat_bf16(BwdEncArgs a) {
  constexpr int KL = KOperand<D>::kLen;
  constexpr int DB = D / 16;
  typedef typename KOperand<D>::T kop_t;
  __shared__ __attribute__((aligned(16))) __bf16 sKt[2][D * kBwdTT];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int j = blockIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const int64_t n0 = (int64_t)j * a.chunk, n1 = min((int64_t)a.N, n0 + a.chunk);
  const int64_t qo = (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off;

  kop_t qh[2], ql[2], dov[2], dol[2];
  float na[2], nd[2];
  bool tv[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = 2 * w + t, m = 16 * i + l16;
    tv[t] = 16 * i < a.Mp;
    const bool real = m < a.M;
    qh[t] = ql[t] = dov[t] = dol[t] = kop_t{};
    if (tv[t]) {
      qh[t] = *reinterpret_cast<const kop_t*>(a.qhi + qo + (int64_t)m * D + KL * g);
      ql[t] = *reinterpret_cast<const kop_t*>(a.qlo + qo + (int64_t)m * D + KL * g);
      dov[t] = *reinterpret_cast<const kop_t*>(a.dor + (lbh * a.Mp + m) * D + KL * g);
      dol[t] = *reinterpret_cast<const kop_t*>(a.dorl + (lbh * a.Mp + m) * D + KL * g);
    }
    na[t] = real ? -a.lse[lbh * a.Mp + m] : -INFINITY;
    nd[t] = real ? -a.delta[lbh * a.Mp + m] : 0.0f;
  }
  f32x4 dqt[2][DB];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int db = 0; db < DB; ++db) dqt[t][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const __bf16* Kh = a.K + bh * (int64_t)a.N * D;
  const __bf16* Vh = a.V + bh * (int64_t)a.N * D;
  // the next step's K and V are loaded while this one computes
  kop_t kn[2], vn[2];
  auto load_kv = [&](int64_t tb) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      kn[hh] = tok_operand<D>(Kh, tb + 16 * hh, n1, l16, g);
      vn[hh] = tok_operand<D>(Vh, tb + 16 * hh, n1, l16, g);
    }
  };
  if (n0 < n1) load_kv(n0);
  int buf = 0;
  for (int64_t tb = n0; tb < n1; tb += 32, buf ^= 1) {
    kop_t ka[2], va[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      ka[hh] = kn[hh];
      va[hh] = vn[hh];
    }
    if (tb + 32 < n1) load_kv(tb + 32);
    if (w == 0) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < KL; ++e) sKt[buf][(KL * g + e) * kBwdTT + 16 * hh + l16] = ka[hh][e];
    }
    __syncthreads();
    bf16x8 kt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) kt[db] = tr_operand(&sKt[buf][(16 * db + l16) * kBwdTT], 0, g);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (!tv[t]) continue;
      f32x4 dl[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f32x4 L = KOperand<D>::mma(ka[hh], qh[t], splat4(na[t]));
        L = KOperand<D>::mma(ka[hh], ql[t], L);
        f32x4 dp = KOperand<D>::mma(va[hh], dov[t], splat4(nd[t]));
        dp = KOperand<D>::mma(va[hh], dol[t], dp);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool live = tb + 16 * hh + 4 * g + r < n1;
          dl[hh][r] = live ? fast_exp2(L[r]) * dp[r] : 0.0f;
        }
      }
      const bf16x8 lb = pack_tiles(dl[0], dl[1]);
#pragma unroll
      for (int db = 0; db < DB; ++db) dqt[t][db] = mfma_k32(kt[db], lb, dqt[t][db]);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int m = 16 * (2 * w + t) + l16;
    if (!tv[t] || m >= a.M) continue;
    float* rec = a.part + ((lbh * a.Mp + m) * a.J + j) * (int64_t)D;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(rec + 16 * db + 4 * g) = dqt[t][db] * a.s;
  }
}

// Arguments of the decode passes (stage 3): keys Qd (c Qd hi/lo rows, Qd^T),
// values Z through Z' = Z - mean Z (hi/lo rows, Z'^T), upstream dY.
struct BwdDecArgs {
  const __bf16* qhi;  // [G][Mp][D]
  const __bf16* qlo;
  const __bf16* qdt;  // [G][D][Mt]
  const __bf16* zh;   // [G][Mp][D]
  const __bf16* zl;
  const __bf16* zt;   // [G][D][Mt]
  const __bf16* K;    // B x H x N x D
  const float* dY;    // B x H x N x D
  float* dK;          // token pass: written
  float* tA;          // [G][tstride] decode log-sum-exp A_n (token pass writes, latent pass reads)
  float* tD;          // [G][tstride] <dY_n, Y'_n>
  int64_t tstride;    // N rounded up to a multiple of 4
  float* part;        // latent pass: [G][Mp][J][2 D], dQd at 0, dZ at D
  int J, chunk, tchunk;
  int N, M, Mp, Mt;
  int64_t bh0;
  float s;
};

// ---- decode token pass: per 32-token block, first A_n and Y'_n with an
// online max over the latent blocks (L = (c Qd) K^T, rows latents), then
// dL = 2^(L - A_n) (Z' dY^T - <dY_n, Y'_n>) and dK^T += Qd^T dL.
template <int D>
__global__ __launch_bounds__(512) void bwd_dec_tok_bf16(BwdDecArgs a) {
  constexpr int KL = KOperand<D>::kLen;
  constexpr int DB = D / 16;
  typedef typename KOperand<D>::T kop_t;
  __shared__ __attribute__((aligned(16))) __bf16 sQh[kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQl[kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sZh[kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sZl[kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQt[D * kBwdTS];
  __shared__ __attribute__((aligned(16))) __bf16 sZt[D * kBwdTS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int Mt = a.Mt, nkb = Mt / 32;
  stage_rows<D>(sQh, a.qhi + lbh * a.Mp * D, a.Mp, Mt, tid, 512);
  stage_rows<D>(sQl, a.qlo + lbh * a.Mp * D, a.Mp, Mt, tid, 512);
  stage_rows<D>(sZh, a.zh + lbh * a.Mp * D, a.Mp, Mt, tid, 512);
  stage_rows<D>(sZl, a.zl + lbh * a.Mp * D, a.Mp, Mt, tid, 512);
  stage_tr<D>(sQt, a.qdt + lbh * (int64_t)D * Mt, Mt, tid, 512);
  stage_tr<D>(sZt, a.zt + lbh * (int64_t)D * Mt, Mt, tid, 512);
  __syncthreads();

  const int64_t n0 = (int64_t)blockIdx.x * a.tchunk, n1 = min((int64_t)a.N, n0 + a.tchunk);
  const __bf16* Kh = a.K + bh * (int64_t)a.N * D;
  const float* Gh = a.dY + bh * (int64_t)a.N * D;
  // K and dY of the next 32-token block are loaded while this one computes
  kop_t kn[2];
  DyRaw<D> yn[2];
  auto load_blk = [&](int64_t tb) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      kn[u] = tok_operand<D>(Kh, tb + 16 * u, n1, l16, g);
      yn[u].load(Gh, tb + 16 * u, n1, l16, g);
    }
  };
  if (n0 + 32 * w < n1) load_blk(n0 + 32 * w);
  for (int64_t tb = n0 + 32 * w; tb < n1; tb += 256) {
    kop_t kb_op[2], gb_op[2], gl_op[2];
    f32x4 gy[2][DB];  // dY_n elements 16 db + 4 g .. + 3, n = tb + 16 u + l16
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      kb_op[u] = kn[u];
      split_hilo<D>(yn[u].x0, yn[u].x1, gb_op[u], gl_op[u]);
#pragma unroll
      for (int db = 0; db < DB; ++db) gy[u][db] = yn[u].y[db];
    }
    if (tb + 256 < n1) load_blk(tb + 256);
    // pass 1: running max, weight sums and Y'^T
    float mrun[2] = {-INFINITY, -INFINITY}, lam[2] = {0.0f, 0.0f};
    f32x4 yt[2][DB];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) yt[u][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int kb = 0; kb < nkb; ++kb) {
      f32x4 L[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int m0 = 32 * kb + 16 * t;
        const kop_t qh = *reinterpret_cast<const kop_t*>(sQh + (m0 + l16) * D + KL * g);
        const kop_t ql = *reinterpret_cast<const kop_t*>(sQl + (m0 + l16) * D + KL * g);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
          L[t][u] = KOperand<D>::mma(qh, kb_op[u], z);
          L[t][u] = KOperand<D>::mma(ql, kb_op[u], L[t][u]);
#pragma unroll
          for (int r = 0; r < 4; ++r) L[t][u][r] = m0 + 4 * g + r < a.M ? L[t][u][r] : -INFINITY;
        }
      }
      bf16x8 zt[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) zt[db] = tr_operand(sZt + (16 * db + l16) * kBwdTS, 32 * kb, g);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float mx = fmaxf(max3(L[0][u][0], L[0][u][1], L[0][u][2]), max3(L[0][u][3], L[1][u][0], L[1][u][1]));
        mx = max_over_rows(fmaxf(mx, fmaxf(L[1][u][2], L[1][u][3])));
        const float mnew = fmaxf(mrun[u], mx);
        const float sc = fast_exp2(mrun[u] - mnew);
        mrun[u] = mnew;
        f32x4 P0, P1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          P0[r] = fast_exp2(L[0][u][r] - mnew);
          P1[r] = fast_exp2(L[1][u][r] - mnew);
        }
        lam[u] = lam[u] * sc + ((P0[0] + P0[1]) + (P0[2] + P0[3])) + ((P1[0] + P1[1]) + (P1[2] + P1[3]));
        const bf16x8 pb = pack_tiles(P0, P1);
#pragma unroll
        for (int db = 0; db < DB; ++db) yt[u][db] = mfma_k32(zt[db], pb, yt[u][db] * sc);
      }
    }
    float nA[2], nDl[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float lt = sum_over_rows(lam[u]);
      float dd = 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) dd = fmaf(gy[u][db][r], yt[u][db][r], dd);
      dd = sum_over_rows(dd) / lt;
      nA[u] = -(mrun[u] + __builtin_log2f(lt));
      nDl[u] = -dd;
      const int64_t n = tb + 16 * u + l16;
      if (g == 0 && n < n1) {
        a.tA[lbh * a.tstride + n] = -nA[u];
        a.tD[lbh * a.tstride + n] = dd;
      }
    }
    // pass 2: dL and dK^T += Qd^T dL
    f32x4 dkt[2][DB];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) dkt[u][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int kb = 0; kb < nkb; ++kb) {
      f32x4 dL[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int m0 = 32 * kb + 16 * t;
        const kop_t qh = *reinterpret_cast<const kop_t*>(sQh + (m0 + l16) * D + KL * g);
        const kop_t ql = *reinterpret_cast<const kop_t*>(sQl + (m0 + l16) * D + KL * g);
        const kop_t zh = *reinterpret_cast<const kop_t*>(sZh + (m0 + l16) * D + KL * g);
        const kop_t zl = *reinterpret_cast<const kop_t*>(sZl + (m0 + l16) * D + KL * g);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          f32x4 L = KOperand<D>::mma(qh, kb_op[u], splat4(nA[u]));
          L = KOperand<D>::mma(ql, kb_op[u], L);
          f32x4 dp = KOperand<D>::mma(zh, gb_op[u], splat4(nDl[u]));
          dp = KOperand<D>::mma(zl, gb_op[u], dp);
          dp = KOperand<D>::mma(zh, gl_op[u], dp);
#pragma unroll
          for (int r = 0; r < 4; ++r) dL[t][u][r] = m0 + 4 * g + r < a.M ? fast_exp2(L[r]) * dp[r] : 0.0f;
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 qt = tr_operand(sQt + (16 * db + l16) * kBwdTS, 32 * kb, g);
#pragma unroll
        for (int u = 0; u < 2; ++u) dkt[u][db] = mfma_k32(qt, pack_tiles(dL[0][u], dL[1][u]), dkt[u][db]);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t n = tb + 16 * u + l16;
      if (n < n1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
          *reinterpret_cast<f32x4*>(a.dK + (bh * (int64_t)a.N + n) * D + 16 * db + 4 * g) = dkt[u][db] * a.s;
      }
    }
  }
}

// ---- decode latent pass: split partials of dZ_m = sum_n P_nm dY_n and
// dQd_m = s sum_n dL_nm K_n, with P_nm = 2^(L - A_n) from the token pass's
// A_n and dL = P (<dY_n, Z'_m> - <dY_n, Y'_n>).  Per 32-token step: L^T =
// K (c Qd)^T, dP'^T = dY Z'^T (rows tokens, cols latents); dZ^T += dY^T P^T
// and dQd^T += K^T dL^T from transposed LDS copies of the step's K and dY.
template <int D>
__global__ __launch_bounds__(512) void bwd_dec_lat_bf16(BwdDecArgs a) {
  constexpr int KL = KOperand<D>::kLen;
  constexpr int DB = D / 16;
  typedef typename KOperand<D>::T kop_t;
  __shared__ __attribute__((aligned(16))) __bf16 sKt[2][D * kBwdTT];
  __shared__ __attribute__((aligned(16))) __bf16 sGt[2][D * kBwdTT];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int j = blockIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int64_t n0 = (int64_t)j * a.chunk, n1 = min((int64_t)a.N, n0 + a.chunk);

  kop_t qh[2], ql[2], zh[2], zl[2];
  bool tv[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = 2 * w + t, m = 16 * i + l16;
    tv[t] = 16 * i < a.Mp;
    qh[t] = ql[t] = zh[t] = zl[t] = kop_t{};
    if (tv[t]) {
      const int64_t o = (lbh * a.Mp + m) * D + KL * g;
      qh[t] = *reinterpret_cast<const kop_t*>(a.qhi + o);
      ql[t] = *reinterpret_cast<const kop_t*>(a.qlo + o);
      zh[t] = *reinterpret_cast<const kop_t*>(a.zh + o);
      zl[t] = *reinterpret_cast<const kop_t*>(a.zl + o);
    }
  }
  f32x4 dzt[2][DB], dqt[2][DB];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int db = 0; db < DB; ++db) dzt[t][db] = dqt[t][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const __bf16* Kh = a.K + bh * (int64_t)a.N * D;
  const float* Gh = a.dY + bh * (int64_t)a.N * D;
  // per-token statistics of the head: rows of a.tstride floats (a multiple
  // of 4, so a lane's four tokens are one aligned 16-byte load)
  const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(a.tA + lbh * a.tstride, (uint32_t)(a.tstride * 4));
  const __amdgpu_buffer_rsrc_t rD = buffer_rsrc(a.tD + lbh * a.tstride, (uint32_t)(a.tstride * 4));
  // the next step's K, dY and statistics are loaded while this one computes
  kop_t kn[2];
  DyRaw<D> yn[2];
  f32x4 an[2], dn[2];
  auto load_step = [&](int64_t tb) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      kn[hh] = tok_operand<D>(Kh, tb + 16 * hh, n1, l16, g);
      yn[hh].load(Gh, tb + 16 * hh, n1, l16, g);
      an[hh] = buffer_load<f32x4>(rA, (int)(tb + 16 * hh + 4 * g) * 4);
      dn[hh] = buffer_load<f32x4>(rD, (int)(tb + 16 * hh + 4 * g) * 4);
    }
  };
  if (n0 < n1) load_step(n0);
  int buf = 0;
  for (int64_t tb = n0; tb < n1; tb += 32, buf ^= 1) {
    kop_t ka[2], ga[2], gl[2];
    f32x4 na[2], nd[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      ka[hh] = kn[hh];
      split_hilo<D>(yn[hh].x0, yn[hh].x1, ga[hh], gl[hh]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool live = tb + 16 * hh + 4 * g + r < n1;
        na[hh][r] = live ? -an[hh][r] : -INFINITY;
        nd[hh][r] = live ? -dn[hh][r] : 0.0f;
      }
    }
    if (tb + 32 < n1) load_step(tb + 32);
    if (w == 0) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < KL; ++e) sKt[buf][(KL * g + e) * kBwdTT + 16 * hh + l16] = ka[hh][e];
    } else if (w == 1) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < KL; ++e) sGt[buf][(KL * g + e) * kBwdTT + 16 * hh + l16] = ga[hh][e];
    }
    __syncthreads();
    bf16x8 kt[DB], gt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      kt[db] = tr_operand(&sKt[buf][(16 * db + l16) * kBwdTT], 0, g);
      gt[db] = tr_operand(&sGt[buf][(16 * db + l16) * kBwdTT], 0, g);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (!tv[t]) continue;
      f32x4 P[2], dl[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f32x4 L = KOperand<D>::mma(ka[hh], qh[t], na[hh]);
        L = KOperand<D>::mma(ka[hh], ql[t], L);
        f32x4 dp = KOperand<D>::mma(ga[hh], zh[t], nd[hh]);
        dp = KOperand<D>::mma(ga[hh], zl[t], dp);
        dp = KOperand<D>::mma(gl[hh], zh[t], dp);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          P[hh][r] = fast_exp2(L[r]);  // 2^-inf = 0 past the split
          dl[hh][r] = P[hh][r] * dp[r];
        }
      }
      const bf16x8 pb = pack_tiles(P[0], P[1]);
      const bf16x8 lb = pack_tiles(dl[0], dl[1]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dzt[t][db] = mfma_k32(gt[db], pb, dzt[t][db]);
        dqt[t][db] = mfma_k32(kt[db], lb, dqt[t][db]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int m = 16 * (2 * w + t) + l16;
    if (!tv[t] || m >= a.M) continue;
    float* rec = a.part + ((lbh * a.Mp + m) * a.J + j) * (int64_t)(2 * D);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      *reinterpret_cast<f32x4*>(rec + 16 * db + 4 * g) = dqt[t][db] * a.s;
      *reinterpret_cast<f32x4*>(rec + D + 16 * db + 4 * g) = dzt[t][db];
    }
  }
}

}  // namespace flarepp

// Backward of the route for bf16 inputs on the matrix cores: the gradients
// dS, dK, dV (float32) of a scalar loss given dY (float32).  The chain rule
// is the one of the float32 path (backward_f32.h): for an SDPA application
// O = SDPA(Q, K, V, s) with P_ij = softmax_j(s <Q_i, K_j>) and upstream dO,
//     dV_j += sum_i P_ij dO_i,   dL_ij = P_ij (<dO_i, V_j> - <dO_i, O_i>),
//     dQ_i += s sum_j dL_ij K_j, dK_j  += s sum_i dL_ij Q_i,
// taken through the decode (queries = tokens, keys = Qd, values = Z), the
// encode and the seed encode (FLARE summary, "Основной механизм FLARE").
//
// Each stage has a latent pass (a workgroup owns one split of the tokens and
// all latents, wave w latents 32 w .. 32 w + 31, and writes split partials
// that bwd_reduce sums) and token-side work (a workgroup owns tokens and
// walks all latents, whose operands it stages in LDS once): the decode's in
// one pass that also forms the per-token statistics the decode's latent pass
// needs, both encode stages' in one final pass, so dK and dV (float32, the
// largest arrays of the call) are read and written once there.  Every
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
// registers (common.h).  Latent operands are staged in LDS as rows with
// XOR-swizzled 16-byte chunks (the route's encode tile layout, slot_off), so
// both the row operand and the transposed one (ds_read_b64_tr_b16) read
// without bank conflicts; the latent passes stream their token operands
// through LDS tiles of the same layout (LatTiles).
#pragma once

#include "common.h"
#include "encode_bf16.h"

namespace flarepp {

constexpr int kBwdBf16MaxM = 256;

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
  __shared__ float spart[256 / D][D];
  const int k = blockIdx.x, tid = threadIdx.x;
  auto load = [&](int m, int d) -> float {
    const int64_t i = (int64_t)k * a.src_blk + (int64_t)m * D + d;
    return a.src_bf16 ? (float)static_cast<const __bf16*>(a.src)[i] : static_cast<const float*>(a.src)[i];
  };
  if (a.center) {
    // column sums: 256 / D threads per column take every (256 / D)-th row,
    // then one thread per column adds their sums in order
    constexpr int P = 256 / D;
    const int d = tid % D, q = tid / D;
    float s = 0.0f;
    for (int m = q; m < a.M; m += P) s += load(m, d);
    spart[q][d] = s;
    __syncthreads();
    if (tid < D) {
      float t = 0.0f;
#pragma unroll
      for (int i = 0; i < P; ++i) t += spart[i][tid];
      smean[tid] = t / (float)a.M;
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

// Arguments of the encode-stage latent pass (stages 1 and 2): queries Q
// (c Q as bf16 hi/lo rows; (b, h)'s block at b * sb + h * sh - off, which
// also covers the seed blocks of stage 1), dO (bf16 hi/lo rows), the
// forward's per-latent log-sum-exp A_m and delta_m = <dO_m, O_m>.
struct BwdEncArgs {
  const __bf16* qhi;
  const __bf16* qlo;
  int64_t q_sb, q_sh, q_off;  // in [.][Mp][D] blocks
  const __bf16* dor;          // [G][Mp][D] dO as bf16 hi
  const __bf16* dorl;         // [G][Mp][D] bf16 lo (dO - hi)
  const float* lse;           // [G][Mp]
  const float* delta;         // [G][Mp]
  const __bf16* K;            // B x H x N x D
  const __bf16* V;
  float* part;                // [G][Mp][J][D]
  int J, chunk;               // token splits
  int H, N, M, Mp;
  int64_t bh0;
  float s;
};

// weights of two C tiles (rows 4 g .. 4 g + 3 of tiles 0 and 1) as the k slots
// of one operand
__device__ __forceinline__ bf16x8 pack_tiles(f32x4 x0, f32x4 x1) {
  const bf16x2 p0 = pack_bf16(x0[0], x0[1]), p1 = pack_bf16(x0[2], x0[3]);
  const bf16x2 p2 = pack_bf16(x1[0], x1[1]), p3 = pack_bf16(x1[2], x1[3]);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ f32x4 splat4(float x) { return f32x4{x, x, x, x}; }

// Row-major [Mp][D] bf16 block -> LDS rows 0 .. Mt - 1 (zero past Mp), the
// 16-byte chunks of row m swizzled as in the encode's tiles (slot_off).
template <int D>
__device__ __forceinline__ void stage_rows(__bf16* dst, const __bf16* src, int Mp, int Mt, int tid, int nthr) {
  constexpr int CH = D / 8;
  for (int e = tid; e < Mt * CH; e += nthr) {
    const int m = e / CH, c = e - m * CH;
    bf16x8 v = bf16x8{};
    if (m < Mp) v = reinterpret_cast<const bf16x8*>(src)[e];
    *reinterpret_cast<bf16x8*>(dst + m * D + ((c ^ chunk_swz<D>(m)) << 3)) = v;
  }
}
// Row operand of latent rows m0 .. m0 + 15 (lane: row m0 + l16, elements KL g ..)
template <int D>
__device__ __forceinline__ typename KOperand<D>::T row_operand(const __bf16* sX, int m0, int l16, int g) {
  return *reinterpret_cast<const typename KOperand<D>::T*>(sX + slot_off<D>(m0 + l16, KOperand<D>::kLen * g));
}
// Transposed operand of latents 32 kb .. 32 kb + 31, elements 16 db .. 16 db + 15
// (lane: row element 16 db + l16, k slots latents 32 kb + 4 g .. + 3 and
// 32 kb + 16 + 4 g .. + 3): two transposing reads, each giving four latents
// of one element when the 16 lanes of a row group supply a 4-latent x
// 16-element block (lane r: latent + r / 4, elements + 4 (r % 4) .. + 3).
template <int D>
__device__ __forceinline__ bf16x8 tr_rows(const __bf16* sX, int kb, int db, int l16, int g) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const __bf16* a0 = sX + slot_off<D>(32 * kb + 4 * g + (l16 >> 2), 16 * db + 4 * (l16 & 3));
  const bf16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a0);
  const bf16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0 + 16 * D));
  return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
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
// dS of the seed blocks from per-head totals src ([G][M][D], the launch's
// heads): out[blk] += sum of src over the heads that use seed block blk
// (every head when the seeds are shared), in head order.
struct BwdSeedSumArgs {
  const float* src;
  float* out;  // [seed_blocks][M][D]
  int M, G, H, seed_blocks;
  int64_t bh0;
};

template <int D>
__global__ __launch_bounds__(256) void bwd_seed_sum(BwdSeedSumArgs a) {
  const int64_t per = (int64_t)a.M * D;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.seed_blocks * per) return;
  const int blk = (int)(i / per);
  const int64_t e = i - blk * per;
  float acc = 0.0f;
  for (int lbh = 0; lbh < a.G; ++lbh) {
    if (a.seed_blocks > 1 && (int)((a.bh0 + lbh) % a.H) != blk) continue;
    acc += a.src[lbh * per + e];
  }
  a.out[i] += acc;
}

// ---- encode-stage token pass, both encode stages at once: dV_n and dK_n
// of the workgroup's tokens (dK added to the decode's part).  Wave w takes
// 32-token blocks tb = n0 + 32 w + 256 i; per stage and 32-latent block kb:
// L = (c Q) K^T - A (rows latents, cols tokens), dP = dO V^T - delta,
// P = 2^L, dL = P dP, then dV^T += dO^T P and dK^T += (c Q)^T dL, the
// transposed operands read from the same LDS rows; dK is scaled by s / c.
struct BwdStageOps {
  const __bf16* qhi;  // c Q as bf16 hi/lo rows; (b, h)'s block at b * q_sb + h * q_sh - q_off
  const __bf16* qlo;
  int64_t q_sb, q_sh, q_off;
  const __bf16* dor;   // [G][Mp][D] dO as bf16 hi
  const __bf16* dorl;  // [G][Mp][D] bf16 lo
  const float* lse;    // [G][Mp] A_m
  const float* delta;  // [G][Mp] <dO_m, O_m>
};

struct BwdEncTokArgs {
  BwdStageOps st[2];  // the encode (queries Qd) and the seed encode (queries S)
  const __bf16* K;
  const __bf16* V;
  float* dK;          // B x H x N x D, holds the decode's part
  float* dV;          // B x H x N x D, written
  int tchunk;         // tokens per workgroup (multiple of 256)
  int H, N, M, Mp, Mt;
  int64_t bh0;
  float kscale;       // s / c (0 when s = 0)
};

template <int D>
__global__ __launch_bounds__(512) void bwd_enc_tok_bf16(BwdEncTokArgs a) {
  constexpr int DB = D / 16;
  typedef typename KOperand<D>::T kop_t;
  __shared__ __attribute__((aligned(16))) __bf16 sQh[2][kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQl[2][kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sDo[2][kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sDol[2][kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) float sNA[2][kBwdBf16MaxM];
  __shared__ __attribute__((aligned(16))) float sND[2][kBwdBf16MaxM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const int Mt = a.Mt, nkb = Mt / 32;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const BwdStageOps& o = a.st[x];
    const int64_t qo = (int64_t)b * o.q_sb + (int64_t)h * o.q_sh - o.q_off;
    stage_rows<D>(sQh[x], o.qhi + qo, a.Mp, Mt, tid, 512);
    stage_rows<D>(sQl[x], o.qlo + qo, a.Mp, Mt, tid, 512);
    stage_rows<D>(sDo[x], o.dor + lbh * a.Mp * D, a.Mp, Mt, tid, 512);
    stage_rows<D>(sDol[x], o.dorl + lbh * a.Mp * D, a.Mp, Mt, tid, 512);
    for (int m = tid; m < Mt; m += 512) {
      const bool real = m < a.M;
      sNA[x][m] = real ? -o.lse[lbh * a.Mp + m] : -INFINITY;
      sND[x][m] = real ? -o.delta[lbh * a.Mp + m] : 0.0f;
    }
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
    for (int x = 0; x < 2; ++x) {
      const __bf16* qh_s = sQh[x];
      const __bf16* ql_s = sQl[x];
      const __bf16* do_s = sDo[x];
      const __bf16* dl_s = sDol[x];
      for (int kb = 0; kb < nkb; ++kb) {
        f32x4 P[2][2], dL[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int m0 = 32 * kb + 16 * t;
          const kop_t qh = row_operand<D>(qh_s, m0, l16, g);
          const kop_t ql = row_operand<D>(ql_s, m0, l16, g);
          const kop_t dov = row_operand<D>(do_s, m0, l16, g);
          const kop_t dol = row_operand<D>(dl_s, m0, l16, g);
          const f32x4 na = *reinterpret_cast<const f32x4*>(&sNA[x][m0 + 4 * g]);
          const f32x4 nd = *reinterpret_cast<const f32x4*>(&sND[x][m0 + 4 * g]);
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
          const bf16x8 dot = tr_rows<D>(do_s, kb, db, l16, g);
          const bf16x8 qt = tr_rows<D>(qh_s, kb, db, l16, g);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            dvt[u][db] = mfma_k32(dot, pb[u], dvt[u][db]);
            dkt[u][db] = mfma_k32(qt, lb[u], dkt[u][db]);
          }
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
          *reinterpret_cast<f32x4*>(a.dK + o) = *reinterpret_cast<const f32x4*>(a.dK + o) + dkt[u][db] * a.kscale;
          *reinterpret_cast<f32x4*>(a.dV + o) = dvt[u][db];
        }
      }
    }
  }
}

// ---- token tiles of the latent passes.  A workgroup streams its split's
// tokens through LDS in tiles of TT = 4096 / D tokens: NOP bf16 operands of
// 8 KB each ([TT][D] rows with the encode tile's chunk swizzle, so the row
// operand and the transposing read are both free of bank conflicts); NF
// float32 operands, staged row-major and split by the waves into a bf16 hi
// and a bf16 lo tile of the same swizzled layout (x = hi + lo to 16 bits);
// and, with STATS, two float rows of TT (the decode's per-token A_n and
// <dY_n, Y'_n>).  Three slots: the barrier that opens tile u is taken after
// every wave has finished tile u - 1, and right after it the loads of tile
// u + 2 go into the slot tile u - 1 held, so two tiles are in flight while
// one is read.  The loads go straight to LDS (dma16), each wave waits for its
// own (and splits its own float32 chunks) before the barrier, and no register
// carries a token operand from one step to the next.  Tiles past the split
// re-read its last token (the masks give those zero weight), so every wave
// issues the same loads per tile and the wait counts are constants.
template <int D, int NOP, int NF, bool STATS>
struct LatTiles {
  static constexpr int TT = 4096 / D;               // tokens per tile
  static constexpr int OPE = TT * D;                // bf16 per operand tile (8 KB)
  static constexpr int HL = NOP * OPE;              // hi, lo tiles of float operand f at HL + 2 f OPE (+ OPE)
  static constexpr int F32 = HL + 2 * NF * OPE;     // float32 staging of operand f at F32 + 2 f OPE
  static constexpr int ST = F32 + 2 * NF * OPE;     // statistics rows
  static constexpr int SLOT = ST + (STATS ? 4 * TT : 0);
  static constexpr int NSI = STATS ? TT / 128 : 0;  // 1 KB loads of the statistics
  static constexpr int STEPS = TT / 32;
  static constexpr int NLOAD = NOP + 2 * NF;        // loads per wave and tile (plus the statistics)
};

// Issue wave `wave`'s loads of the tile at token tb into slot `sl`: chunk
// 64 wave + lane of every bf16 operand (lane l of a load fills LDS chunk
// base + 16 l, so it fetches the (token, chunk) the swizzle places there),
// chunks 128 wave .. 128 wave + 127 of every float32 operand (row-major);
// waves below NSI also load 1 KB of the [A | D] statistics rows.
template <int D, int NOP, int NF, bool STATS>
__device__ __forceinline__ void lat_tile_dma(__bf16* sl, const __bf16* const* src, const float* const* srcf,
                                             const float* tA, const float* tD, int64_t tb, int64_t n1, int wave,
                                             int lane) {
  typedef LatTiles<D, NOP, NF, STATS> T;
  constexpr int U = D / 8;
  const int c = wave * 64 + lane;
  const int t = c / U;
  const int u = (c % U) ^ chunk_swz<D>(t);
  const int64_t row = min(tb + t, n1 - 1);
#pragma unroll
  for (int o = 0; o < NOP; ++o) dma16(src[o] + row * D + 8 * u, sl + o * T::OPE + wave * 512);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cf = wave * 128 + i * 64 + lane;
      const int64_t rf = min(tb + cf / (D / 4), n1 - 1);
      dma16(reinterpret_cast<const __bf16*>(srcf[f] + rf * D + 4 * (cf % (D / 4))),
            sl + T::F32 + 2 * f * T::OPE + (wave * 128 + i * 64) * 8);
    }
  }
  if (STATS && wave < T::NSI) {
    const bool isA = 4 * c < T::TT;
    const int64_t tok = min(tb + (isA ? 4 * c : 4 * c - T::TT), (n1 - 1) & ~int64_t(3));
    dma16(reinterpret_cast<const __bf16*>((isA ? tA : tD) + tok), sl + T::ST + wave * 512);
  }
}

// Wait until this wave's loads of the oldest tile in flight (slot `sl`) have
// landed (those of the next tile may still be in flight), split its float32
// chunks into the hi/lo tiles, then open the tile to the workgroup.  The lgkm
// wait makes this wave's LDS writes land, and its reads of the previous tile
// complete, before the barrier.
template <int D, int NOP, int NF, bool STATS>
__device__ __forceinline__ void lat_tile_open(__bf16* sl, int wave, int lane) {
  typedef LatTiles<D, NOP, NF, STATS> T;
  if (STATS && wave < T::NSI)
    FLAREPP_WAIT_VM(T::NLOAD + 1);
  else
    FLAREPP_WAIT_VM(T::NLOAD);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cf = wave * 128 + i * 64 + lane;
      const f32x4 x = *reinterpret_cast<const f32x4*>(sl + T::F32 + 2 * f * T::OPE + cf * 8);
      const bf16x2 h0 = pack_bf16(x[0], x[1]), h1 = pack_bf16(x[2], x[3]);
      const bf16x2 l0 = pack_bf16(x[0] - (float)h0[0], x[1] - (float)h0[1]);
      const bf16x2 l1 = pack_bf16(x[2] - (float)h1[0], x[3] - (float)h1[1]);
      const int o = slot_off<D>(cf / (D / 4), 4 * (cf % (D / 4)));
      *reinterpret_cast<bf16x4*>(sl + T::HL + 2 * f * T::OPE + o) = bf16x4{h0[0], h0[1], h1[0], h1[1]};
      *reinterpret_cast<bf16x4*>(sl + T::HL + 2 * f * T::OPE + T::OPE + o) = bf16x4{l0[0], l0[1], l1[0], l1[1]};
    }
  }
  __builtin_amdgcn_s_waitcnt(kEncWaitLgkm0);
  ring_barrier();
}

// Transposed operand of a 32-token step from a tile (lane: row element
// 16 db + l16, k slots tokens 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3):
// p = step base + slot_off(4 g + l16 / 4, 16 db + 4 (l16 % 4)).
template <int D>
__device__ __forceinline__ bf16x8 tr_at(const __bf16* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const bf16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  const bf16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 16 * D));
  return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}

// ---- encode-stage latent pass: split partials of dQ_m = s sum_n dL_mn K_n.
// Compiled for four waves per SIMD (at most 128 VGPRs; 48 KB of LDS), so two
// workgroups share a CU.
// Per 32-token step: L^T = K (c Q)^T - A (rows tokens, cols latents),
// dP^T = V dO^T - delta, dL = 2^L dP (zero past the split), dQ^T += K^T dL^T,
// K and V from the LDS tiles (K^T through transposing reads).
template <int D>
__global__ __launch_bounds__(512, 4) void bwd_enc_lat_bf16(BwdEncArgs a) {
  constexpr int KL = KOperand<D>::kLen;
  constexpr int DB = D / 16;
  typedef typename KOperand<D>::T kop_t;
  typedef LatTiles<D, 2, 0, false> T;
  __shared__ __attribute__((aligned(16))) __bf16 ring[3 * T::SLOT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // the latent operands must not be counted with the tiles' loads
  FLAREPP_WAIT_VM(0);

  const __bf16* const src[2] = {a.K + bh * (int64_t)a.N * D, a.V + bh * (int64_t)a.N * D};
  const int ko = slot_off<D>(l16, KL * g);
  int to[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) to[db] = slot_off<D>(4 * g + (l16 >> 2), 16 * db + 4 * (l16 & 3));

  const int64_t ntiles = n1 > n0 ? (n1 - n0 + T::TT - 1) / T::TT : 0;
  if (ntiles > 0) {
    lat_tile_dma<D, 2, 0, false>(ring, src, nullptr, nullptr, nullptr, n0, n1, w, lane);
    lat_tile_dma<D, 2, 0, false>(ring + T::SLOT, src, nullptr, nullptr, nullptr, n0 + T::TT, n1, w, lane);
  }
  int cur = 0;
  for (int64_t u = 0; u < ntiles; ++u) {
    lat_tile_open<D, 2, 0, false>(ring + cur * T::SLOT, w, lane);
    const int nxt = cur == 0 ? 2 : cur - 1;
    lat_tile_dma<D, 2, 0, false>(ring + nxt * T::SLOT, src, nullptr, nullptr, nullptr, n0 + (u + 2) * T::TT, n1, w,
                                 lane);
    const __bf16* sK = ring + cur * T::SLOT;
    const __bf16* sV = sK + T::OPE;
    const int64_t tb0 = n0 + u * T::TT;
    const int nsteps = (int)min<int64_t>(T::STEPS, (n1 - tb0 + 31) / 32);
#pragma unroll 1
    for (int st = 0; st < nsteps; ++st) {
      const int64_t tb = tb0 + 32 * st;
      const int so = 32 * st * D;
      kop_t ka[2], va[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        ka[hh] = *reinterpret_cast<const kop_t*>(sK + so + 16 * hh * D + ko);
        va[hh] = *reinterpret_cast<const kop_t*>(sV + so + 16 * hh * D + ko);
      }
      bf16x8 kt[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) kt[db] = tr_at<D>(sK + so + to[db]);
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
          if (tb + 32 <= n1) {
#pragma unroll
            for (int r = 0; r < 4; ++r) dl[hh][r] = fast_exp2(L[r]) * dp[r];
          } else {  // the split's last, partial step
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const bool live = tb + 16 * hh + 4 * g + r < n1;
              dl[hh][r] = live ? fast_exp2(L[r]) * dp[r] : 0.0f;
            }
          }
        }
        const bf16x8 lb = pack_tiles(dl[0], dl[1]);
#pragma unroll
        for (int db = 0; db < DB; ++db) dqt[t][db] = mfma_k32(kt[db], lb, dqt[t][db]);
      }
    }
    cur = cur == 2 ? 0 : cur + 1;
  }
  // the trailing tiles' loads must land before the workgroup's LDS is released
  FLAREPP_WAIT_VM(0);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int m = 16 * (2 * w + t) + l16;
    if (!tv[t] || m >= a.M) continue;
    float* rec = a.part + ((lbh * a.Mp + m) * a.J + j) * (int64_t)D;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(rec + 16 * db + 4 * g) = dqt[t][db] * a.s;
  }
}

// Arguments of the decode passes (stage 3): keys Qd (c Qd hi/lo rows),
// values Z through Z' = Z - mean Z (hi/lo rows), upstream dY.
struct BwdDecArgs {
  const __bf16* qhi;  // [G][Mp][D] c Qd as bf16 hi/lo
  const __bf16* qlo;
  const __bf16* zh;   // [G][Mp][D] Z' as bf16 hi/lo
  const __bf16* zl;
  const __bf16* K;    // B x H x N x D
  const float* dY;    // [G][N][D] the upstream gradient of the launch's heads
  const float* qnorm; // [G][Mp] ||Qd_m||
  float c;            // s log2 e
  float* dK;          // token pass: written
  float* tA;          // [G][tstride] decode log-sum-exp A_n (token pass writes, latent pass reads)
  float* tD;          // [G][tstride] <dY_n, Y'_n>
  int64_t tstride;    // N rounded up to a multiple of 4
  float* part;        // latent pass: [G][Mp][J][2 D], dQd at 0, dZ at D
  int J, chunk, tchunk;
  int N, M, Mp, Mt;
  int64_t bh0;
  float s;
  float kscale;       // s / c (0 when s = 0)
};

// ---- decode token pass: per 32-token block, first A_n and Y'_n over the
// latent blocks (L = (c Qd) K^T, rows latents), then
// dL = 2^(L - A_n) (Z' dY^T - <dY_n, Y'_n>) and dK^T += (c Qd)^T dL (scaled
// by s / c; the transposed operands read from the LDS rows).  The shift
// of the first pass is the bound mu_n = |c| ||K_n|| max ||Qd_m|| when
// 2 mu_n <= 100 for every token of the wave's block (no max, no rescaling),
// else a running max over the latent blocks.
template <int D>
__global__ __launch_bounds__(512) void bwd_dec_tok_bf16(BwdDecArgs a) {
  constexpr int KL = KOperand<D>::kLen;
  constexpr int DB = D / 16;
  typedef typename KOperand<D>::T kop_t;
  __shared__ __attribute__((aligned(16))) __bf16 sQh[kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQl[kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sZh[kBwdBf16MaxM * D];
  __shared__ __attribute__((aligned(16))) __bf16 sZl[kBwdBf16MaxM * D];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int Mt = a.Mt, nkb = Mt / 32;
  stage_rows<D>(sQh, a.qhi + lbh * a.Mp * D, a.Mp, Mt, tid, 512);
  stage_rows<D>(sQl, a.qlo + lbh * a.Mp * D, a.Mp, Mt, tid, 512);
  stage_rows<D>(sZh, a.zh + lbh * a.Mp * D, a.Mp, Mt, tid, 512);
  stage_rows<D>(sZl, a.zl + lbh * a.Mp * D, a.Mp, Mt, tid, 512);
  float qmax = 0.0f;
  for (int m = lane; m < a.Mp; m += 64) qmax = fmaxf(qmax, a.qnorm[lbh * a.Mp + m]);
  qmax = wave_max(qmax);
  __syncthreads();
  const bool ragged = a.M < Mt;  // the last latent block has padding rows
  // pad rows of latent block kb: rows m0 + 4 g + r >= M take -inf logits
  auto mask_pad = [&](f32x4& L, int m0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) L[r] = m0 + 4 * g + r < a.M ? L[r] : -INFINITY;
  };

  const int64_t n0 = (int64_t)blockIdx.x * a.tchunk, n1 = min((int64_t)a.N, n0 + a.tchunk);
  const __bf16* Kh = a.K + bh * (int64_t)a.N * D;
  const float* Gf = a.dY + lbh * (int64_t)a.N * D;
  // K and dY of the next 32-token block are loaded while this one computes;
  // dY (float32) both as the elements of the lane's operand slots (KL g ..)
  // and as the C-tile elements 16 db + 4 g .. (the same ones when D = 16)
  constexpr int KQ = KL / 4;
  kop_t kn[2];
  f32x4 yn[2][KQ], gyn[2][DB];
  auto load_blk = [&](int64_t tb) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t n = tb + 16 * u;
      kn[u] = tok_operand<D>(Kh, n, n1, l16, g);
      const int64_t cnt = n1 > n ? n1 - n : 0;
      const __amdgpu_buffer_rsrc_t r = buffer_rsrc(Gf + n * D, (uint32_t)(cnt * D * 4));
#pragma unroll
      for (int q = 0; q < KQ; ++q) yn[u][q] = buffer_load<f32x4>(r, (l16 * D + KL * g + 4 * q) * 4);
      if constexpr (D == 32) {
#pragma unroll
        for (int db = 0; db < DB; ++db) gyn[u][db] = buffer_load<f32x4>(r, (l16 * D + 16 * db + 4 * g) * 4);
      }
    }
  };
  if (n0 + 32 * w < n1) load_blk(n0 + 32 * w);
  for (int64_t tb = n0 + 32 * w; tb < n1; tb += 256) {
    kop_t kb_op[2], gb_op[2], gl_op[2];
    f32x4 gy[2][DB];  // dY_n elements 16 db + 4 g .. + 3, n = tb + 16 u + l16
    float mu[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      kb_op[u] = kn[u];
      // dY as a bf16 hi/lo operand pair (x = hi + lo to 16 bits)
#pragma unroll
      for (int e = 0; e < KL; ++e) {
        const float x = yn[u][e / 4][e % 4];
        const __bf16 hi = (__bf16)x;
        gb_op[u][e] = hi;
        gl_op[u][e] = (__bf16)(x - (float)hi);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if constexpr (D == 32)
          gy[u][db] = gyn[u][db];
        else
          gy[u][db] = yn[u][0];
      }
      float k2 = 0.0f;
#pragma unroll
      for (int e = 0; e < KL; ++e) k2 = fmaf((float)kb_op[u][e], (float)kb_op[u][e], k2);
      mu[u] = fabsf(a.c) * __builtin_sqrtf(sum_over_rows(k2)) * qmax * (1.0f + 1.0f / 4096.0f);
    }
    if (tb + 256 < n1) load_blk(tb + 256);
    const bool bounded = __all(2.0f * fmaxf(mu[0], mu[1]) <= 100.0f);

    // pass 1: weight sums and Y'^T
    float mrun[2], lam[2] = {0.0f, 0.0f};
    f32x4 yt[2][DB];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      mrun[u] = bounded ? mu[u] : -INFINITY;
#pragma unroll
      for (int db = 0; db < DB; ++db) yt[u][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    for (int kb = 0; kb < nkb; ++kb) {
      f32x4 L[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int m0 = 32 * kb + 16 * t;
        const kop_t qh = row_operand<D>(sQh, m0, l16, g);
        const kop_t ql = row_operand<D>(sQl, m0, l16, g);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          L[t][u] = KOperand<D>::mma(qh, kb_op[u], splat4(bounded ? -mu[u] : 0.0f));
          L[t][u] = KOperand<D>::mma(ql, kb_op[u], L[t][u]);
          if (ragged && kb == nkb - 1) mask_pad(L[t][u], m0);
        }
      }
      bf16x8 zt[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) zt[db] = tr_rows<D>(sZh, kb, db, l16, g);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x4 P0, P1;
        if (bounded) {  // logits already shifted by mu
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            P0[r] = fast_exp2(L[0][u][r]);
            P1[r] = fast_exp2(L[1][u][r]);
          }
          lam[u] += ((P0[0] + P0[1]) + (P0[2] + P0[3])) + ((P1[0] + P1[1]) + (P1[2] + P1[3]));
          const bf16x8 pb = pack_tiles(P0, P1);
#pragma unroll
          for (int db = 0; db < DB; ++db) yt[u][db] = mfma_k32(zt[db], pb, yt[u][db]);
        } else {  // running max
          float mx = fmaxf(max3(L[0][u][0], L[0][u][1], L[0][u][2]), max3(L[0][u][3], L[1][u][0], L[1][u][1]));
          mx = max_over_rows(fmaxf(mx, fmaxf(L[1][u][2], L[1][u][3])));
          const float mnew = fmaxf(mrun[u], mx);
          const float sc = fast_exp2(mrun[u] - mnew);
          mrun[u] = mnew;
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
        const kop_t qh = row_operand<D>(sQh, m0, l16, g);
        const kop_t ql = row_operand<D>(sQl, m0, l16, g);
        const kop_t zh = row_operand<D>(sZh, m0, l16, g);
        const kop_t zl = row_operand<D>(sZl, m0, l16, g);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          f32x4 L = KOperand<D>::mma(qh, kb_op[u], splat4(nA[u]));
          L = KOperand<D>::mma(ql, kb_op[u], L);
          if (ragged && kb == nkb - 1) mask_pad(L, m0);
          f32x4 dp = KOperand<D>::mma(zh, gb_op[u], splat4(nDl[u]));
          dp = KOperand<D>::mma(zl, gb_op[u], dp);
          dp = KOperand<D>::mma(zh, gl_op[u], dp);
#pragma unroll
          for (int r = 0; r < 4; ++r) dL[t][u][r] = fast_exp2(L[r]) * dp[r];
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 qt = tr_rows<D>(sQh, kb, db, l16, g);
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
          *reinterpret_cast<f32x4*>(a.dK + (bh * (int64_t)a.N + n) * D + 16 * db + 4 * g) = dkt[u][db] * a.kscale;
      }
    }
  }
}

// ---- decode latent pass: split partials of dZ_m = sum_n P_nm dY_n and
// dQd_m = s sum_n dL_nm K_n, with P_nm = 2^(L - A_n) from the token pass's
// A_n and dL = P (<dY_n, Z'_m> - <dY_n, Y'_n>).  Per 32-token step: L^T =
// K (c Qd)^T, dP'^T = dY Z'^T (rows tokens, cols latents); dZ^T += dY^T P^T
// and dQd^T += K^T dL^T; K, dY (split into hi and lo in LDS) and the
// statistics come from the LDS tiles, K^T and dY^T through transposing reads.
template <int D>
__global__ __launch_bounds__(512) void bwd_dec_lat_bf16(BwdDecArgs a) {
  constexpr int KL = KOperand<D>::kLen;
  constexpr int DB = D / 16;
  typedef typename KOperand<D>::T kop_t;
  typedef LatTiles<D, 1, 1, true> T;
  __shared__ __attribute__((aligned(16))) __bf16 ring[3 * T::SLOT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // the latent operands must not be counted with the tiles' loads
  FLAREPP_WAIT_VM(0);

  const __bf16* const src[1] = {a.K + bh * (int64_t)a.N * D};
  const float* const srcf[1] = {a.dY + lbh * (int64_t)a.N * D};
  const float* tA = a.tA + lbh * a.tstride;
  const float* tD = a.tD + lbh * a.tstride;
  const int ko = slot_off<D>(l16, KL * g);
  int to[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) to[db] = slot_off<D>(4 * g + (l16 >> 2), 16 * db + 4 * (l16 & 3));

  const int64_t ntiles = n1 > n0 ? (n1 - n0 + T::TT - 1) / T::TT : 0;
  if (ntiles > 0) {
    lat_tile_dma<D, 1, 1, true>(ring, src, srcf, tA, tD, n0, n1, w, lane);
    lat_tile_dma<D, 1, 1, true>(ring + T::SLOT, src, srcf, tA, tD, n0 + T::TT, n1, w, lane);
  }
  int cur = 0;
  for (int64_t u = 0; u < ntiles; ++u) {
    lat_tile_open<D, 1, 1, true>(ring + cur * T::SLOT, w, lane);
    const int nxt = cur == 0 ? 2 : cur - 1;
    lat_tile_dma<D, 1, 1, true>(ring + nxt * T::SLOT, src, srcf, tA, tD, n0 + (u + 2) * T::TT, n1, w, lane);
    const __bf16* sK = ring + cur * T::SLOT;
    const __bf16* sGh = sK + T::HL;
    const __bf16* sGl = sK + T::HL + T::OPE;
    const float* sA = reinterpret_cast<const float*>(sK + T::ST);
    const float* sD = sA + T::TT;
    const int64_t tb0 = n0 + u * T::TT;
    const int nsteps = (int)min<int64_t>(T::STEPS, (n1 - tb0 + 31) / 32);
#pragma unroll 1
    for (int st = 0; st < nsteps; ++st) {
      const int64_t tb = tb0 + 32 * st;
      const int so = 32 * st * D;
      kop_t ka[2], ga[2], gl[2];
      f32x4 na[2], nd[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        ka[hh] = *reinterpret_cast<const kop_t*>(sK + so + 16 * hh * D + ko);
        ga[hh] = *reinterpret_cast<const kop_t*>(sGh + so + 16 * hh * D + ko);
        gl[hh] = *reinterpret_cast<const kop_t*>(sGl + so + 16 * hh * D + ko);
        const f32x4 av = *reinterpret_cast<const f32x4*>(sA + 32 * st + 16 * hh + 4 * g);
        const f32x4 dv = *reinterpret_cast<const f32x4*>(sD + 32 * st + 16 * hh + 4 * g);
        if (tb + 32 <= n1) {
          na[hh] = -av;
          nd[hh] = -dv;
        } else {  // the split's last, partial step
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool live = tb + 16 * hh + 4 * g + r < n1;
            na[hh][r] = live ? -av[r] : -INFINITY;
            nd[hh][r] = live ? -dv[r] : 0.0f;
          }
        }
      }
      bf16x8 kt[DB], gt[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        kt[db] = tr_at<D>(sK + so + to[db]);
        gt[db] = tr_at<D>(sGh + so + to[db]);
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
    cur = cur == 2 ? 0 : cur + 1;
  }
  // the trailing tiles' loads must land before the workgroup's LDS is released
  FLAREPP_WAIT_VM(0);
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

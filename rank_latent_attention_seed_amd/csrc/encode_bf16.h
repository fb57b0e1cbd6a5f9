// Split-N encode on bf16 matrix cores: for one (b, h), one split of the N
// tokens and up to 256 latents, compute the partial softmax statistics of
//     O_m = sum_n softmax_n(s <Q_m, K_n>) V_n
// i.e. a running max mu_m (log2 units), a sum lambda_m and an unnormalised
// accumulator acc_m[D].  It serves both encode calls of the route: the seed
// encode (Q = the latent seeds; FLARE++ abstract, the extra encode call) and
// FLARE's encode (Q = the synthesised queries; FLARE summary, "Основной
// механизм FLARE", encode step).  Splits are combined exactly by the merge
// kernel from these statistics, as the pages' token-sharded implementation
// combines per-device latent outputs with their softmax statistics (French
// technical summary, "Contributions Clés", multi-GPU context parallelism).
//
// Work decomposition.  A workgroup of NW waves (4 or 8) owns one (b, h,
// split, latent group); each wave owns MBW 16-latent blocks and all share
// tiles of TN tokens of K and V.  Tiles travel HBM -> LDS by direct-to-LDS
// loads (no staging registers) through a ring of two slots: the loads of the
// next tile are issued right after the barrier that opens the current one,
// so one tile is in flight while one is read (a tile is several microseconds
// of work, far longer than its loads take); the tile loop is unrolled by two
// so every slot address is static.  16-byte chunks of each token row are
// XOR-swizzled in LDS (the fetching lane picks the chunk that belongs to its
// slot) so the matrix-core operand reads are free of bank conflicts
// (chunk_swz).  Per 32-token step a wave reads the step's K and V operands
// and, for each of its latent blocks in turn, computes S^T = K Q^T tiles
// (rows = tokens, cols = latents), turns them into softmax weights in
// registers, and accumulates O^T += V^T P^T; V's operand comes from the
// token-major tile through transposing LDS reads (ds_read_b64_tr_b16).
// There is no software pipeline across blocks: that keeps a wave within 128
// registers, so two eight-wave workgroups (64 KB of ring each) share a CU
// and four waves per SIMD hide each other's matrix-core, exponential and
// LDS latencies (measured 7% faster than a two-wave-per-SIMD kernel that
// pipelined the blocks within each wave).
//
// Softmax arithmetic.  A synthesised query (Qd, float32) arrives
// pre-multiplied by c = s * log2(e) as a bf16 hi/lo pair (two MFMAs per
// tile, ~16 mantissa bits), and -mu_m enters as the MFMA accumulator input,
// so the tile is already t = c <Q_m, K_n> - mu_m; in the route's bounded
// encode, heads within the fp16 logit bound (f16_logits, common.h) take c Q
// as one fp16 operand against keys converted to fp16 in the ring instead
// (one product per tile).  The seeds are bf16 inputs
// and therefore an exact operand (EXQ): one MFMA per tile gives <S_m, K_n>
// to float32 rounding, and one FMA per score applies c and the shift (four
// matrix-core products per 32-token step of a wave traded for sixteen VALU
// operations, which measured faster over the whole route).  A weight is one
// exp2.  mu_m is either
//   * a bound: |c| ||Q_m|| max_n ||K_n|| (Cauchy-Schwarz), supplied by the
//     caller when it is known and keeps every exponent within [-100, 0]; no
//     per-score max is taken; or
//   * online: initialised from the first step's exact column max and raised
//     only when some value in a step exceeds mu_m + TAU (exp2(TAU) keeps
//     every weight and sum finite), at which point acc and lambda are
//     rescaled and the step's scores recomputed against the new shift.  Both give the same softmax up to rounding (softmax is
//     invariant to a common shift).
// lambda_m sums the same rounded weights that enter the PV product (computed
// on the matrix core as a row of ones times P^T).  The encodes with a running
// max form the PV product in fp16, the bound-shifted one in bf16 (see Pv).
#pragma once

#include "common.h"

namespace flarepp {

struct EncodeArgs {
  const __bf16* q_hi;  // pre-scaled query operand rows, padded to Mp (zero rows beyond M)
  const __bf16* q_lo;  // low part of the same
  int64_t q_sb, q_sh;  // element strides of the operand between batches / heads
  int64_t q_off;       // the operand rows of (b, h) start at b*q_sb + h*q_sh - q_off
  // Alternatively (q_seed non-null, the kernels compiled with EXQ) the
  // unscaled bf16 query rows [.][M][D], with the same (b, h) addressing: an
  // exact operand (rows at or past M zero) whose products are scaled by qc
  // in float32.
  const __bf16* q_seed;
  float qc;
  int M;
  const __bf16* K;     // B x H x N x D
  const __bf16* V;     // B x H x N x D
  float* part;         // [G][Mp][J][D + 4] partial records (G = heads of this launch)
  float* knorm;        // [G][J] max squared key norm of each split, or null
  const float* bias;   // [G][Mp] mu_m bound (log2 units; +inf = use online), or null
  // Bounded encodes of the route: the seed encode's split key norms ([G][Jk],
  // squared) and the latent norms ||Qd_m|| (the operand's block layout over
  // D), from which the head's logit bound picks the fp16 logit form; or null
  const float* kin;
  const float* qnorm;
  int Jk;
  int H, N, Mp, J, chunk;
  int64_t bh0;         // first (b, h) of this launch: grid.y = lbh indexes (b, h) = bh0 + lbh
};

template <int D>
struct KOperand;
template <>
struct KOperand<32> {
  typedef bf16x8 T;
  static constexpr int kLen = 8;
  __device__ __forceinline__ static f32x4 mma(T a, T b, f32x4 c) { return mfma_k32(a, b, c); }
};
template <>
struct KOperand<16> {
  typedef bf16x4 T;
  static constexpr int kLen = 4;
  __device__ __forceinline__ static f32x4 mma(T a, T b, f32x4 c) { return mfma_k16(a, b, c); }
};

// Number format of the P V product (the weights and the value tile on the
// matrix core).  bf16 has float32's exponent range and an 8-bit significand.
// fp16, used by the encodes that take a running max, has an 11-bit
// significand, so each weight's rounding error is a quarter of bf16's; that
// error is what limits the seed encode's Qd, and the later stages amplify an
// error in Qd by about |s| ||K|| (Qd is their query, and the decode's key).
// fp16's range (largest finite 65504, subnormals down to 2^-24) is kept by
// the running max: the largest weight of a split is at least 1, so a weight
// that flushes to zero is below 2^-24 of it (a split of n tokens loses at
// most n 2^-25 of its sum that way); when every step is checked, weights
// stay below 2^8.  Under the tile rule (steps unchecked) a score could still
// exceed the running max by 16 binades; the weight is then infinite, so is
// the split's sum, and the merge recomputes that (latent, split) record from
// K and V (merge.h, refit_record).  The value tile is converted from bf16 in
// LDS by the wave that loaded it.
template <bool F16>
struct Pv {
  typedef bf16x8 T;
};
template <>
struct Pv<true> {
  typedef f16x8 T;
};

// ---- tile geometry and the LDS ring.  A slot holds one tile of K or V
// (TE bf16 = TN tokens x D); the ring has two K slots and two V slots in one
// kernel-local LDS array, the V slot of a tile right after its K slot, so
// that every operand read of a step is a lane base plus an offset that fits
// the instruction's 16-bit immediate.  Eight-wave workgroups use 16 KB slots
// (a 64 KB ring: two workgroups per CU); four-wave workgroups use 8 KB
// slots.
template <int D, int NW>
struct Ring {
  static constexpr int TE = NW == 8 ? 8192 : 4096;  // elements per slot
  static constexpr int TN = TE / D;                 // tokens per tile
  static constexpr int SPT = TN / 32;               // 32-token steps per tile
  static constexpr int DI = TE / 8 / 64 / NW;       // 1 KB loads per wave, operand and tile
  static constexpr int kDma = 2 * DI;               // loads per wave and tile
  static constexpr int SLOTS = 2;
  template <int I>
  __device__ __forceinline__ static __bf16* k(__bf16* ring) {
    return ring + 2 * I * TE;
  }
  template <int I>
  __device__ __forceinline__ static __bf16* v(__bf16* ring) {
    return ring + (2 * I + 1) * TE;
  }
};

// Swizzle of the 16-byte chunks of token row t (D/8 chunks per row): the
// chunk holding elements 8u..8u+7 sits at position u ^ swz(t).  gfx950's LDS
// has 64 banks of 4 bytes; for D = 32 (64-byte rows) the K operand read
// (ds_read_b128: lane (g, c16) reads chunk g of row c16) and the transposing
// V read (ds_read_b64_tr_b16: 16 lanes read 4 rows x 32 bytes) are both free
// of bank conflicts with swz(t) = (t >> 1) & 3, measured with
// SQ_LDS_BANK_CONFLICT on MI355X (4 and 2 cycles per wave instruction; the
// swizzle (t >> 2) & 3 takes twice as long on both).
template <int D>
__host__ __device__ __forceinline__ constexpr int chunk_swz(int t) {
  return D == 32 ? ((t >> 1) & 3) : ((t >> 3) & 1);
}
// The swizzle of row t equals that of rows t + 16 and t + 32 (the operand
// offsets of encode_tiles rely on it).
template <int D>
constexpr bool swz_step_invariant() {
  for (int t = 0; t < 64; ++t)
    if (chunk_swz<D>(t) != chunk_swz<D>(t + 16) || chunk_swz<D>(t) != chunk_swz<D>(t + 32)) return false;
  return true;
}
static_assert(swz_step_invariant<32>() && swz_step_invariant<16>(), "chunk swizzle must repeat every 16 rows");
// Element offset of (token t, element e) inside a tile slot.
template <int D>
__device__ __forceinline__ int slot_off(int t, int e) {
  return t * D + ((((e >> 3) ^ chunk_swz<D>(t)) << 3) | (e & 7));
}

// s_waitcnt with vmcnt <= n (n < 64); lgkmcnt and expcnt are not waited on.
// The empty asm statements keep the compiler from moving memory accesses
// across the wait.
#define FLAREPP_WAIT_VM(n)                                                                      \
  do {                                                                                          \
    asm volatile("" ::: "memory");                                                              \
    __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | (((n) >> 4) << 14));    \
    asm volatile("" ::: "memory");                                                              \
  } while (0)

// Workgroup barrier without the memory wait that __syncthreads() implies
// (the ring's loads are waited for explicitly, per tile).
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One direct-to-LDS load: every lane fetches 16 bytes from its own global
// address into LDS at lds_base + 16 * lane.  Written as an asm statement (it
// has no register results) so that the compiler does not track the LDS
// write: its own bookkeeping would make every later LDS read of any ring
// slot wait for all loads in flight, which would serialise the ring.  The
// ring's waits are explicit (FLAREPP_WAIT_VM before each tile's barrier).
// M0 (the LDS base of the load) is set and consumed inside the statement; the
// compiler treats M0 as reserved and uses it nowhere else in this library
// (tests/test_kernel_asm.py checks the generated code for that).
__device__ __forceinline__ void dma16(const __bf16* src, const __bf16* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory");
}

// The same load from a wave-uniform base (an SGPR pair) plus a 32-bit byte
// offset per lane: a tile's lane offsets are the same for every tile of a
// split (only the base moves), so they cost no per-tile address arithmetic.
__device__ __forceinline__ void dma16s(const __bf16* base, uint32_t off, const __bf16* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m0) : "memory");
}

// Issue the direct-to-LDS loads of one tile into slot I: the NW waves split
// the tile's 16-byte chunks of K and of V (instructions of 1 KB each); lane l
// of an instruction fills LDS chunk base + 16 l and therefore fetches the
// (token, chunk) that the swizzle places there.  Tokens past the split
// re-read the split's last row (they receive zero weight), so every tile
// issues the same number of loads and the wait counts stay uniform.
template <int D, int NW, int I>
__device__ __forceinline__ void tile_dma(__bf16* ring, const __bf16* Kp, const __bf16* Vp, int tb, int n1,
                                         int wave, int lane) {
  typedef Ring<D, NW> R;
  constexpr int U = D / 8;
  // the tile's first row as the (uniform) base; rows past the split clamp
  // to its last row only in a split's last, partial tile
  const int64_t base = (int64_t)__builtin_amdgcn_readfirstlane(tb) * D;
  const int last = max(__builtin_amdgcn_readfirstlane(n1 - 1 - tb), 0);  // a tile starts before n1
  const bool partial = last < R::TN - 1;
#pragma unroll
  for (int i = 0; i < R::DI; ++i) {
    const int blk = wave * R::DI + i;
    const int s = blk * 64 + lane;
    const int t = s / U;
    const int u = (s % U) ^ chunk_swz<D>(t);
    const int row = partial ? min(t, last) : t;
    const uint32_t off = (uint32_t)(row * D + 8 * u) * 2u;
    dma16s(Kp + base, off, R::template k<I>(ring) + blk * 512);
    dma16s(Vp + base, off, R::template v<I>(ring) + blk * 512);
  }
}

// Per-wave register state of the encode: query operands, the softmax
// statistics (the shift -mu enters each S^T tile as its accumulator input),
// and O^T.
// acc[DB] is the sum lambda: its tile is ONES^T P^T, whose row 0 carries the
// column sums of the rounded weights (so lambda sums exactly the weights that
// enter O^T).
template <int D, int MBW>
struct EncodeState {
  typedef typename KOperand<D>::T kop_t;
  kop_t qh[MBW], ql[MBW];
  float mu[MBW];
  float qn2[MBW];  // ||c Q_m||^2 of the lane's latent (from the hi + lo operand)
  float c;         // exact query operand: the scale applied to its products
  f32x4 acc[D / 16 + 1][MBW];
};

// K operands (A of S^T = K Q^T: lane holds token row c16, k-chunk g) of step
// ks; ko = slot_off(c16, KL g).
template <int D>
__device__ __forceinline__ void load_kop(const __bf16* sK, int ks, int ko, typename KOperand<D>::T& k0,
                                         typename KOperand<D>::T& k1) {
  typedef typename KOperand<D>::T kop_t;
  const __bf16* b = sK + ks * 32 * D + ko;
  k0 = *reinterpret_cast<const kop_t*>(b);
  // D = 16: the two 8-byte reads are 512 bytes apart, which the compiler would
  // fuse into one ds_read2st64_b64 -- measured on MI355X at 16 LDS cycles per
  // wave instruction where the two ds_read_b64 take 2 each (SQ_LDS_BANK_CONFLICT)
  if (D == 16) asm volatile("" ::: "memory");
  k1 = *reinterpret_cast<const kop_t*>(b + 16 * D);
}

// V^T operands of step ks: lane (row d = 16 db + c16, k-row g) needs V[tok][d]
// for the eight tokens of its k-slots; one transposing read gives a lane four
// tokens of its column when the 16 lanes of row g supply the 4-token x
// 16-column block (lane r: token base + r/4, columns 16 db + 4 (r%4) ..+3).
// With F16 the slot holds the fp16 conversion of the tile (same layout).
// vo[db] = slot_off(4 g + c16 / 4, 16 db + 4 (c16 % 4)).
template <int D, bool F16>
__device__ __forceinline__ void load_vop(const __bf16* sV, int ks, const int (&vo)[D / 16],
                                         typename Pv<F16>::T (&v)[D / 16]) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 h16x4;
  typedef __attribute__((address_space(3))) h16x4 lds_h16x4;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    const __bf16* a0 = sV + ks * 32 * D + vo[db];
    const __bf16* a1 = a0 + 16 * D;
    if constexpr (F16) {
      const f16x4 v0 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h16x4*)a0));
      const f16x4 v1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h16x4*)a1));
      v[db] = f16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    } else {
      const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a0);
      const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a1);
      v[db] = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
  }
}

// Form of the query operand (LQ): kHiLo, c Q as a bf16 hi/lo pair; kExact,
// the exact bf16 query rows (the seeds), whose products are scaled by c in
// float32; kF16, c Q in fp16 against keys converted to fp16 in the ring
// (f16_logits).
constexpr int kHiLo = 0, kExact = 1, kF16 = 2;

// S^T tiles of latent block i: query as hi + lo with the shift as the
// accumulator input, or (kExact) the exact query rows in one product whose
// float32 result is scaled and shifted, t = c <Q_m, K_n> - mu_m, or (kF16)
// one fp16 product with the shift as the accumulator input (qh holds the
// fp16 bits of c Q, the key slot the fp16 keys).
template <int D, int MBW, int LQ>
__device__ __forceinline__ void block_logits(const EncodeState<D, MBW>& st, int i, typename KOperand<D>::T k0,
                                             typename KOperand<D>::T k1, f32x4& s0, f32x4& s1) {
  if constexpr (LQ == kF16) {
    typedef typename KOperand16<D>::T hop_t;
    const f32x4 cb = f32x4{-st.mu[i], -st.mu[i], -st.mu[i], -st.mu[i]};
    const hop_t q = __builtin_bit_cast(hop_t, st.qh[i]);
    s0 = KOperand16<D>::mma(__builtin_bit_cast(hop_t, k0), q, cb);
    s1 = KOperand16<D>::mma(__builtin_bit_cast(hop_t, k1), q, cb);
  } else if constexpr (LQ == kExact) {
    const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
    s0 = KOperand<D>::mma(k0, st.qh[i], z);
    s1 = KOperand<D>::mma(k1, st.qh[i], z);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s0[r] = fmaf(s0[r], st.c, -st.mu[i]);
      s1[r] = fmaf(s1[r], st.c, -st.mu[i]);
    }
  } else {
    const f32x4 cb = f32x4{-st.mu[i], -st.mu[i], -st.mu[i], -st.mu[i]};
    s0 = KOperand<D>::mma(k0, st.qh[i], cb);
    s1 = KOperand<D>::mma(k1, st.qh[i], cb);
    s0 = KOperand<D>::mma(k0, st.ql[i], s0);
    s1 = KOperand<D>::mma(k1, st.ql[i], s1);
  }
}

template <bool F16>
__device__ __forceinline__ typename Pv<F16>::T weights(f32x4 s0, f32x4 s1) {
  if constexpr (F16) {
    const f16x2 p0 = pack_f16(fast_exp2(s0[0]), fast_exp2(s0[1]));
    const f16x2 p1 = pack_f16(fast_exp2(s0[2]), fast_exp2(s0[3]));
    const f16x2 p2 = pack_f16(fast_exp2(s1[0]), fast_exp2(s1[1]));
    const f16x2 p3 = pack_f16(fast_exp2(s1[2]), fast_exp2(s1[3]));
    return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  } else {
    const bf16x2 p0 = pack_bf16(fast_exp2(s0[0]), fast_exp2(s0[1]));
    const bf16x2 p1 = pack_bf16(fast_exp2(s0[2]), fast_exp2(s0[3]));
    const bf16x2 p2 = pack_bf16(fast_exp2(s1[0]), fast_exp2(s1[1]));
    const bf16x2 p3 = pack_bf16(fast_exp2(s1[2]), fast_exp2(s1[3]));
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
}

// O^T and lambda updates of block i from its weights p and its step's V^T operands.
template <int D, int MBW, bool F16>
__device__ __forceinline__ void block_update(EncodeState<D, MBW>& st, int i, const typename Pv<F16>::T (&v)[D / 16],
                                             typename Pv<F16>::T p, typename Pv<F16>::T ones) {
#pragma unroll
  for (int db = 0; db < D / 16; ++db) st.acc[db][i] = mfma_k32(v[db], p, st.acc[db][i]);
  st.acc[D / 16][i] = mfma_k32(ones, p, st.acc[D / 16][i]);
}

// One 32-token step (step ks of the tile in K slot sK and V slot sV): the
// step's K and V operands, then each latent block of the wave in turn.
// ONLINE: running max, starting from the exact column max of the split's
// first step and raised lazily (only when a score exceeds mu + TAU, so
// weights and sums stay finite); the raise rescales O^T and lambda and
// recomputes the block's scores against the new shift (cheaper than keeping
// them live, and rare).  Otherwise the shift is a bound.  MASK (the split's
// ragged last step): tokens at or past n1 weigh zero.
template <int D, int MBW, bool F16, bool ONLINE, bool MASK, int LQ>
__device__ __forceinline__ void encode_step(EncodeState<D, MBW>& st, const __bf16* sK, const __bf16* sV, int ks,
                                            int ko, const int (&vo)[D / 16], int sb, int n1, int g,
                                            typename Pv<F16>::T ones) {
  constexpr int DB = D / 16;
  constexpr float TAU = 8.0f;
  typename KOperand<D>::T k0, k1;
  load_kop<D>(sK, ks, ko, k0, k1);
  typename Pv<F16>::T v[DB];
  load_vop<D, F16>(sV, ks, vo, v);
  auto mask = [&](f32x4& s0, f32x4& s1) {
    if (MASK) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (sb + 4 * g + r >= n1) s0[r] = -INFINITY;
        if (sb + 16 + 4 * g + r >= n1) s1[r] = -INFINITY;
      }
    }
  };
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
    f32x4 s0, s1;
    block_logits<D, MBW, LQ>(st, i, k0, k1, s0, s1);
    mask(s0, s1);
    if (ONLINE) {
      const float lm = fmaxf(max3(s1[2], s1[3], max3(s0[3], s1[0], max3(s0[0], s0[1], s0[2]))), s1[1]);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(lm > TAU) != 0, 0)) {
        const float d = fmaxf(max_over_rows(lm), 0.0f);
        st.mu[i] += d;
        const float al = fast_exp2(-d);
#pragma unroll
        for (int db = 0; db <= DB; ++db) st.acc[db][i] *= al;
        block_logits<D, MBW, LQ>(st, i, k0, k1, s0, s1);
        mask(s0, s1);
      }
    }
    const typename Pv<F16>::T p = weights<F16>(s0, s1);
    block_update<D, MBW, F16>(st, i, v, p, ones);
    // keep the next block's work from being hoisted into this one's: the
    // live ranges would no longer fit four waves per SIMD
    if (ONLINE) __builtin_amdgcn_sched_barrier(0);
  }
}

// Largest squared key norm among the tokens of the K tile in slot I whose
// 16-byte chunks this wave loaded itself (the U chunks of one token row are
// loaded by U adjacent lanes, so a quad-permute DPP sum completes each row),
// valid as soon as this wave's loads of the tile have landed; the same value
// in every lane.  Squared norms are +0 or more (or NaN, whose bit pattern
// orders above every finite one and so forces the checked path), so the
// maximum is taken on the bit patterns as unsigned integers, which folds
// each DPP move into its max.
template <int D, int NW, int I>
__device__ __forceinline__ float own_knorm(const __bf16* ring, int wave, int lane) {
  typedef Ring<D, NW> R;
  constexpr int U = D / 8;
  uint32_t best = 0;
#pragma unroll
  for (int i = 0; i < R::DI; ++i) {
    const int blk = wave * R::DI + i;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(R::template k<I>(const_cast<__bf16*>(ring)) + blk * 512 + 8 * lane);
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x2 pr = {x[2 * e], x[2 * e + 1]};
      ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
    }
    ss += dpp<0xB1>(ss);              // quad_perm [1,0,3,2]
    if (U == 4) ss += dpp<0x4E>(ss);  // quad_perm [2,3,0,1]
    best = max(best, __float_as_uint(ss));
  }
  best = max(best, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)best, 0x124, 0xF, 0xF, false));  // row_ror:4
  best = max(best, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)best, 0x128, 0xF, 0xF, false));  // row_ror:8
  const auto s1 = __builtin_amdgcn_permlane16_swap(best, best, false, false);
  best = max(s1[0], s1[1]);
  const auto s2 = __builtin_amdgcn_permlane32_swap(best, best, false, false);
  return __uint_as_float(max(s2[0], s2[1]));
}

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt not waited on).
constexpr uint32_t kEncWaitLgkm0 = 0xF | (0x7 << 4) | (0x3 << 14);

// Ring protocol (two slots).  Tile u+1's loads are issued right after the
// barrier that opens tile u (when the split has a tile u+1); before that barrier a wave waits for its own
// loads of tile u (the only ones in flight), so every wave's part of tile u
// has landed once all have arrived.  The barrier opening tile u is taken
// after the wave's last step of tile u-1, so the slot refilled right after
// it, (u+1) & 1, held tile u-1, which every wave has finished reading.
//
// Work a wave does on its own chunks of tile u (slot I) once they have
// landed, published by the barrier that opens the tile:
//   TNORM: the largest squared key norm of its rows, stored in
//     sKm[u & 1][wave]; after the barrier every wave takes the maximum over
//     the NW entries.  Two buffers suffice: the entries of tile u are read
//     right after the barrier that opens it, and rewritten (for tile u + 2)
//     only after the next barrier.
//   F16: the fp16 conversion of its value chunks, in place.
//   KF16: the fp16 conversion of its key chunks, in place (after TNORM's
//     norms, which read the bf16 keys; the two are not combined).
// It runs in ring_open, after the wave's wait for its loads of tile u.
template <int D, int NW, int I, bool TNORM, bool F16, bool KF16>
__device__ __forceinline__ void tile_prep(__bf16* ring, float* sKm, int u, int wave, int lane) {
  typedef Ring<D, NW> R;
  static_assert(!(TNORM && KF16), "key norms read the bf16 keys");
  if (F16) {
#pragma unroll
    for (int i = 0; i < R::DI; ++i) {
      __bf16* c = R::template v<I>(ring) + (wave * R::DI + i) * 512 + 8 * lane;
      *reinterpret_cast<f16x8*>(c) = to_f16<f16x8>(*reinterpret_cast<const bf16x8*>(c));
    }
  }
  if (KF16) {
#pragma unroll
    for (int i = 0; i < R::DI; ++i) {
      __bf16* c = R::template k<I>(ring) + (wave * R::DI + i) * 512 + 8 * lane;
      *reinterpret_cast<f16x8*>(c) = to_f16<f16x8>(*reinterpret_cast<const bf16x8*>(c));
    }
  }
  if (TNORM) {
    const float part = own_knorm<D, NW, I>(ring, wave, lane);
    if (lane == 0) sKm[(u & 1) * NW + wave] = part;
  }
}

template <int D, int NW, int I, bool TNORM, bool F16, bool KF16>
__device__ __forceinline__ float ring_open(__bf16* ring, float* sKm, const __bf16* Kp, const __bf16* Vp, int u,
                                           int n0, int n1, bool more, int wave, int lane) {
  typedef Ring<D, NW> R;
  FLAREPP_WAIT_VM(0);
  float* slot = sKm + (u & 1) * NW;
  tile_prep<D, NW, I, TNORM, F16, KF16>(ring, sKm, u, wave, lane);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kEncWaitLgkm0);  // this wave's LDS accesses are done before the barrier
  ring_barrier();
  if (more) tile_dma<D, NW, I ^ 1>(ring, Kp, Vp, n0 + (u + 1) * R::TN, n1, wave, lane);
  float km2 = 0.0f;
  if (TNORM) {
    km2 = slot[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) km2 = fmaxf(km2, slot[w]);
  }
  return km2;
}

// Tile rule of the online path.  A score of latent m in a tile is at most
// ||c Q_m|| max_n ||K_n|| - mu_m (Cauchy-Schwarz, log2 units, maximum over
// the tile's tokens); when that bound is at most TAU_SKIP for every latent of
// the wave, no weight of the tile can exceed 2^TAU_SKIP (sums stay far from
// the float range), and the per-step comparison with the running max is
// skipped for the whole tile.  Otherwise (or for non-finite norms) every
// step checks.
template <int D, int MBW>
__device__ __forceinline__ bool tile_needs_check(const EncodeState<D, MBW>& st, float km2) {
  constexpr float TAU_SKIP = 32.0f;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
    // ||c Q_m|| sqrt(km2) <= mu_m + TAU_SKIP, squared (both sides >= 0)
    const float lim = st.mu[i] + TAU_SKIP;
    bad |= !(lim >= 0.0f && st.qn2[i] * km2 <= lim * lim);
  }
  return __builtin_amdgcn_ballot_w64(bad) != 0;
}

// Tile t in slot I: open it (except tile 0, opened before the running max
// is seeded), then its steps.  With TNORM, km2 is the largest squared key
// norm of tile t once it is open.
template <int D, int NW, int MBW, bool F16, bool KNORM, bool ONLINE, bool SKIP, int LQ, int I>
__device__ __forceinline__ void encode_tile(EncodeState<D, MBW>& st, __bf16* ring, float* sKm, const __bf16* Kp,
                                            const __bf16* Vp, int t, int ntiles, int n0, int n1, int wave, int lane,
                                            bool wave_active, int g, int ko, const int (&vo)[D / 16],
                                            typename Pv<F16>::T ones, float& km2, float& kn2) {
  typedef Ring<D, NW> R;
  constexpr bool TNORM = KNORM || (ONLINE && SKIP);
  if (t > 0)
    km2 = ring_open<D, NW, I, TNORM, F16, LQ == kF16>(ring, sKm, Kp, Vp, t, n0, n1, t + 1 < ntiles, wave, lane);
  if (KNORM) kn2 = fmaxf(kn2, km2);
  if (!wave_active) return;
  const int tb = n0 + t * R::TN;
  const int nsteps = min(R::SPT, (n1 - tb + 31) / 32);
  const int full = tb + nsteps * 32 <= n1 ? nsteps : nsteps - 1;  // steps with no token past n1
  const __bf16* sK = R::template k<I>(ring);
  const __bf16* sV = R::template v<I>(ring);
  if (ONLINE && (!SKIP || tile_needs_check<D, MBW>(st, km2))) {
#pragma unroll 1
    for (int ks = 0; ks < full; ++ks)
      encode_step<D, MBW, F16, true, false, LQ>(st, sK, sV, ks, ko, vo, tb + 32 * ks, n1, g, ones);
    if (full < nsteps) encode_step<D, MBW, F16, true, true, LQ>(st, sK, sV, full, ko, vo, tb + 32 * full, n1, g, ones);
  } else {
#pragma unroll 1
    for (int ks = 0; ks < full; ++ks)
      encode_step<D, MBW, F16, false, false, LQ>(st, sK, sV, ks, ko, vo, tb + 32 * ks, n1, g, ones);
    if (full < nsteps) encode_step<D, MBW, F16, false, true, LQ>(st, sK, sV, full, ko, vo, tb + 32 * full, n1, g, ones);
  }
}

// SKIP: the online path applies the tile rule (tile_needs_check); otherwise
// every step of the online path checks.
template <int D, int NW, int MBW, bool F16, bool KNORM, bool ONLINE, bool SKIP, int LQ>
__device__ __forceinline__ void encode_tiles(EncodeState<D, MBW>& st, __bf16* ring, float* sKm, const __bf16* Kp,
                                             const __bf16* Vp, int n0, int n1, int wave, int lane,
                                             bool wave_active, int g, int c16, float& kn2) {
  typedef Ring<D, NW> R;
  constexpr int DB = D / 16;
  constexpr bool TNORM = KNORM || (ONLINE && SKIP);
  const int ntiles = (n1 - n0 + R::TN - 1) / R::TN;
  typedef typename Pv<F16>::T pv_t;
  // A operand of the lambda tile: row 0 all ones
  pv_t ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = c16 == 0 ? 1.0f : 0.0f;
  // this lane's operand offsets (elements) within a step of a slot: K row c16
  // at element KL g, and per 16-column block db the V^T read of row
  // 4 g + c16 / 4 at element 16 db + 4 (c16 % 4).  The rows 16 further on, and
  // every later step (32 rows on), add constants: the swizzle of a row depends
  // on bits of its index that neither changes (chunk_swz).
  const int ko = slot_off<D>(c16, KOperand<D>::kLen * g);
  int vo[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) vo[db] = slot_off<D>(4 * g + (c16 >> 2), 16 * db + 4 * (c16 & 3));

  tile_dma<D, NW, 0>(ring, Kp, Vp, n0, n1, wave, lane);
  float km2 = ring_open<D, NW, 0, TNORM, F16, LQ == kF16>(ring, sKm, Kp, Vp, 0, n0, n1, ntiles > 1, wave, lane);
  if (wave_active && ONLINE) {
    // the running max starts at the exact column max of the first step
    // (the shift is still zero here)
    typename KOperand<D>::T k0, k1;
    load_kop<D>(R::template k<0>(ring), 0, ko, k0, k1);
#pragma unroll
    for (int i = 0; i < MBW; ++i) {
      f32x4 s0, s1;
      block_logits<D, MBW, LQ>(st, i, k0, k1, s0, s1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (n0 + 4 * g + r >= n1) s0[r] = -INFINITY;
        if (n0 + 16 + 4 * g + r >= n1) s1[r] = -INFINITY;
      }
      const float lm = fmaxf(max3(s1[2], s1[3], max3(s0[3], s1[0], max3(s0[0], s0[1], s0[2]))), s1[1]);
      st.mu[i] = max_over_rows(lm);
    }
  }
  for (int t = 0; t < ntiles; t += 2) {
    encode_tile<D, NW, MBW, F16, KNORM, ONLINE, SKIP, LQ, 0>(st, ring, sKm, Kp, Vp, t, ntiles, n0, n1, wave, lane, wave_active,
                                                          g, ko, vo, ones, km2, kn2);
    if (t + 1 >= ntiles) break;
    encode_tile<D, NW, MBW, F16, KNORM, ONLINE, SKIP, LQ, 1>(st, ring, sKm, Kp, Vp, t + 1, ntiles, n0, n1, wave, lane,
                                                          wave_active, g, ko, vo, ones, km2, kn2);
  }
  // the ring's trailing loads must land before the workgroup's LDS is released
  FLAREPP_WAIT_VM(0);
}

// BOUNDED: the shift may come from a.bias (the bound path, with the online
// path as fallback when a bound is unsafe); otherwise always online.  F16: the
// P V product in fp16 (online encodes only: the bound shift does not keep the
// weights inside fp16's range).  Eight-wave workgroups are compiled for four
// waves per SIMD (at most 128 VGPRs), so two of them share a CU.
template <int D, int NW, int MBW, bool KNORM, bool BOUNDED, bool F16, bool EXQ>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 4 : 2) void encode_split_bf16(EncodeArgs a) {
  static_assert(!(F16 && BOUNDED), "fp16 weights need the running max");
  static_assert(!(EXQ && BOUNDED), "the bound shift comes with the synthesised queries' hi/lo operand");
  constexpr int DB = D / 16;     // 16-row blocks of O^T
  constexpr int KL = KOperand<D>::kLen;
  typedef typename KOperand<D>::T kop_t;
  __shared__ __attribute__((aligned(16))) __bf16 ring[2 * Ring<D, NW>::SLOTS * Ring<D, NW>::TE];
  __shared__ float sKm[2 * NW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4, c16 = lane & 15;
  const int j = blockIdx.x;
  const int64_t lbh = blockIdx.y, bh = a.bh0 + lbh;
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const int n0 = j * a.chunk;
  const int n1 = min(a.N, n0 + a.chunk);
  const int nMB = a.Mp >> 4;
  const int mb0 = (blockIdx.z * NW + wave) * MBW;
  const bool wave_active = mb0 < nMB;

  const __bf16* Kp = a.K + bh * (int64_t)a.N * D;
  const __bf16* Vp = a.V + bh * (int64_t)a.N * D;

  // ---- query operands (B of S^T = K Q^T: lane holds column m, k = d) and shift
  EncodeState<D, MBW> st;
  st.c = a.qc;
  bool need_online = !BOUNDED || a.bias == nullptr;
  {
    const int64_t qo = (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off;
#pragma unroll
    for (int i = 0; i < MBW; ++i) {
      const int mblk = mb0 + i;
      if (mblk < nMB) {
        const int m = mblk * 16 + c16;
        if constexpr (EXQ) {
          kop_t x = kop_t{};
          if (m < a.M) x = *reinterpret_cast<const kop_t*>(a.q_seed + qo + (int64_t)m * D + KL * g);
          st.qh[i] = x;
          st.ql[i] = kop_t{};
        } else {
          st.qh[i] = *reinterpret_cast<const kop_t*>(a.q_hi + qo + (int64_t)m * D + KL * g);
          st.ql[i] = *reinterpret_cast<const kop_t*>(a.q_lo + qo + (int64_t)m * D + KL * g);
        }
        st.mu[i] = (BOUNDED && a.bias) ? a.bias[lbh * a.Mp + m] : 0.0f;
      } else {
        st.qh[i] = kop_t{};
        st.ql[i] = kop_t{};
        st.mu[i] = 0.0f;
      }
      need_online |= !(st.mu[i] <= 1e30f);
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < KL; ++e) {
        const float x = EXQ ? a.qc * (float)st.qh[i][e] : (float)st.qh[i][e] + (float)st.ql[i][e];
        ss = fmaf(x, x, ss);
      }
      st.qn2[i] = sum_over_rows(ss);
#pragma unroll
      for (int db = 0; db <= DB; ++db) st.acc[db][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // The route's bounded encode: the head's logit bound mu_g (the same rule
  // and inputs as the decode's) picks the fp16 logit form for the whole
  // workgroup (every wave reads the same norms).  Within it every latent's
  // bound is at most mu_g <= 16, so no wave needs the online path.
  bool q16 = false;
  if constexpr (BOUNDED) {
    if (a.kin && a.qnorm && a.bias) {
      float k2 = 0.0f;
      for (int jj = lane; jj < a.Jk; jj += 64) k2 = fmaxf(k2, a.kin[lbh * a.Jk + jj]);
      const float kmax = __builtin_sqrtf(wave_max(k2));
      const int64_t qo = (int64_t)b * a.q_sb + (int64_t)h * a.q_sh - a.q_off;
      float qmax = 0.0f;
      for (int m = lane; m < a.Mp; m += 64) qmax = fmaxf(qmax, a.qnorm[qo / D + m]);
      qmax = wave_max(qmax);
      q16 = f16_logits(fabsf(a.qc) * kmax * qmax * (1.0f + 1.0f / 4096.0f), kmax, qmax, a.qc);
    }
  }
  const bool online = __any(need_online) && !q16;
#pragma unroll
  for (int i = 0; i < MBW; ++i)
    if (online) st.mu[i] = 0.0f;
  float kn2 = 0.0f;
  // the operand loads above must not be counted with the ring's loads
  FLAREPP_WAIT_VM(0);

  constexpr int LQ = EXQ ? kExact : kHiLo;
  if (!BOUNDED || online) {
    encode_tiles<D, NW, MBW, F16, KNORM, true, !BOUNDED, LQ>(st, ring, sKm, Kp, Vp, n0, n1, wave, lane, wave_active, g,
                                                         c16, kn2);
  } else if constexpr (BOUNDED) {
    if (q16) {
      // c Q as fp16 in the hi slot (hi + lo is exact in float32, rounded once)
#pragma unroll
      for (int i = 0; i < MBW; ++i)
        st.qh[i] = __builtin_bit_cast(kop_t, to_f16<typename KOperand16<D>::T>(st.qh[i], st.ql[i]));
      encode_tiles<D, NW, MBW, false, KNORM, false, false, kF16>(st, ring, sKm, Kp, Vp, n0, n1, wave, lane,
                                                                wave_active, g, c16, kn2);
    } else {
      encode_tiles<D, NW, MBW, false, KNORM, false, false, LQ>(st, ring, sKm, Kp, Vp, n0, n1, wave, lane, wave_active,
                                                           g, c16, kn2);
    }
  }

  // ---- partial records
  if (wave_active) {
    constexpr int PS = Part<D>::kStride;
#pragma unroll
    for (int i = 0; i < MBW; ++i) {
      const int mblk = mb0 + i;
      if (mblk >= nMB) break;
      const int m = mblk * 16 + c16;
      float* rec = a.part + ((lbh * a.Mp + m) * (int64_t)a.J + j) * PS;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(rec + 16 * db + 4 * g) = st.acc[db][i];
      if (g == 0) {
        rec[D] = st.acc[DB][i][0];  // row 0 of the lambda tile
        rec[D + 1] = st.mu[i];
      }
    }
  }
  // kn2 is the maximum of the tile maxima, the same in every lane
  if (KNORM && tid == 0 && blockIdx.z == 0) a.knorm[lbh * a.J + j] = kn2;
}

}  // namespace flarepp

// Device-side building blocks shared by the libflarepp kernels (gfx950 only).
//
// Matrix-core operand layouts (v_mfma_f32_16x16x32_bf16; lane l, g = l / 16):
//   A (16 rows x 32 k): lane holds row l % 16, k = 8g .. 8g + 7
//   B (32 k x 16 cols): lane holds col l % 16, k = 8g .. 8g + 7
//   C (16 x 16 fp32)  : lane holds col l % 16, rows 4g .. 4g + 3
// v_mfma_f32_16x16x16_bf16 is the same with k = 4g .. 4g + 3.
// A C tile of S^T = K Q^T (rows = tokens, cols = latents) therefore leaves each
// lane with one latent and four tokens; two such tiles give exactly the eight
// k-slots of a B operand over 32 tokens, so softmax weights feed the next
// contraction without leaving registers, provided the other operand orders its
// 32 k-slots the same way: slot (g, j) <-> token 4g + j for j < 4 and
// 16 + 4g + (j - 4) for j >= 4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flarepp {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even pair conversions (v_cvt_pk_bf16_f32 and
// v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ bf16x2 pack_bf16(float lo, float hi) {
  bf16x2 r = {(__bf16)lo, (__bf16)hi};
  return r;
}
__device__ __forceinline__ f16x2 pack_f16(float lo, float hi) {
  f16x2 r = {(_Float16)lo, (_Float16)hi};
  return r;
}

// Raw buffer resources: loads whose VGPR offset (plus the instruction offset)
// is at or past num_records bytes return zeros and such stores are dropped
// by the hardware, so a stream that ends mid-block needs no clamped
// addresses or guarded stores.  The range check does not include the scalar
// offset, so every offset that must be checked goes in the VGPR offset (the
// helpers below pass a scalar offset of zero).  Word 3 selects the 32-bit
// data format.
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// 16- or 8-byte load at byte offset off (range-checked).
template <typename T>
__device__ __forceinline__ T buffer_load(__amdgpu_buffer_rsrc_t r, int off) {
  static_assert(sizeof(T) == 16 || sizeof(T) == 8, "16- or 8-byte loads");
  if constexpr (sizeof(T) == 16)
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  else
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// 16-byte store at byte offset off (range-checked).
__device__ __forceinline__ void buffer_store(f32x4 v, __amdgpu_buffer_rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}

// Reductions across the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48),
// i.e. over g for a fixed l % 16: two permlane swaps, no LDS traffic.
__device__ __forceinline__ float max_over_rows(float x) {
  uint32_t u = __float_as_uint(x);
  auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  float y = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  uint32_t v = __float_as_uint(y);
  auto t = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float sum_over_rows(float x) {
  uint32_t u = __float_as_uint(x);
  auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  float y = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  uint32_t v = __float_as_uint(y);
  auto t = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// All-lane reductions over a whole wave using DPP row operations and the
// two permlane swaps (VALU only): quad butterflies, rotations by 4 and 8
// within each 16-lane row, then across rows.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x124>(x);  // row_ror:4
  x += dpp<0x128>(x);  // row_ror:8
  return sum_over_rows(x);
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x124>(x));
  x = fmaxf(x, dpp<0x128>(x));
  return max_over_rows(x);
}

__device__ __forceinline__ float max3(float a, float b, float c) {
  return fmaxf(fmaxf(a, b), c);  // v_max3_f32
}

// Single-product logits.  The keys are exact in fp16 as well as in bf16 when
// |k| < 2^10 (bf16's 8-bit significand fits fp16's 11 bits; below fp16's
// normal range a key moves by at most 2^-25: these kernels run with 16-bit
// denormals kept, float_denorm_mode_16_64 = 3, so nothing flushes to zero).  Rounding c Qd to fp16 moves
// each product term by at most 2^-11 of itself, so a logit by at most
// 2^-11 |c| ||Qd_m|| ||K_n|| <= 2^-11 mu_g (Cauchy-Schwarz), where
// mu_g = |c| max_n ||K_n|| max_m ||Qd_m|| is the head's logit bound.  With
// mu_g <= kF16Logit that is at most 2^-7 in log2 units: a weight changes by at
// most 0.55%, next to the 0.39% of the bf16 rounding every weight takes
// before the weights' own product.  In the route, the encode of stage 2 and
// the decode take one fp16 product per logit tile for the heads within that
// bound, instead of the hi/lo pair; the others keep the pair.
constexpr float kF16Logit = 16.0f;
__device__ __forceinline__ bool f16_logits(float mu_g, float kmax, float qmax, float c) {
  return mu_g <= kF16Logit && kmax <= 1024.0f && fabsf(c) * qmax <= 1024.0f;
}

template <int D>
struct KOperand16;
template <>
struct KOperand16<32> {
  typedef f16x8 T;
  __device__ __forceinline__ static f32x4 mma(T a, T b, f32x4 c) { return mfma_k32(a, b, c); }
};
template <>
struct KOperand16<16> {
  typedef f16x4 T;
  __device__ __forceinline__ static f32x4 mma(T a, T b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};
// fp16 operand from a bf16 one (the key rows), and from a bf16 hi/lo pair
// (c Qd: hi + lo is exact in float32, then rounded to nearest once)
template <typename H, typename B>
__device__ __forceinline__ H to_f16(const B x) {
  H r;
#pragma unroll
  for (int e = 0; e < (int)(sizeof(B) / 2); ++e) r[e] = (_Float16)(float)x[e];
  return r;
}
template <typename H, typename B>
__device__ __forceinline__ H to_f16(const B hi, const B lo) {
  H r;
#pragma unroll
  for (int e = 0; e < (int)(sizeof(B) / 2); ++e) r[e] = (_Float16)((float)hi[e] + (float)lo[e]);
  return r;
}

// Per-split softmax partial record: acc[0..D-1], sum at D, max (log2 units) at
// D+1.  Records are stored [head][latent][split] so that one latent's records
// are contiguous for the merge.
template <int D>
struct Part {
  static constexpr int kStride = D + 4;  // 16-byte aligned records
};

}  // namespace flarepp

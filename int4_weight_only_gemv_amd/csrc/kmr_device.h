// Device-side helpers shared by the kmr kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kmr {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// Cross-lane moves through DPP.  Lanes that a row mask disables read 0.
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, BANK_MASK, true));
}

// Sum over each 16-lane row; every lane of the row receives the row's sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x124>(v);  // row_ror 4
  v += dpp<0x128>(v);  // row_ror 8
  return v;
}

// Value of the lane 8 positions away inside the 16-lane row (i <-> i^8).
__device__ __forceinline__ float row16_swap8(float v) { return dpp<0x128>(v); }

// Sum over the 64-lane wave, returned uniform (from lane 63).
// threadIdx.x behind an empty asm barrier: values derived from it are recomputed
// where they are used instead of being hoisted out of long loops and kept live
// (the persistent kernels run out of registers otherwise).
__device__ __forceinline__ int otid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Marks a loaded value as used here, so that the compiler waits for its load at
// this point (right after a poll, where every earlier load has already
// completed and the wait is free) rather than at its first real use, where the
// wait would also cover loads issued in between.
template <typename T>
__device__ __forceinline__ void settle(T v) {
  asm volatile("" ::"v"(v));
}
__device__ __forceinline__ void settle(uint4 v) {
  settle(v.x);
  settle(v.y);
  settle(v.z);
  settle(v.w);
}

// 2^x with the hardware exponential (about 1 ulp; results below the smallest
// normal float may flush to zero): for softmax and log-sum-exp weights, where such
// terms are negligible against the largest weight of 1.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// 1/sqrt(x) with the hardware reciprocal square root (within 1 ulp); used for
// RMSNorm scales, whose inputs are at least epsilon.
__device__ __forceinline__ float rsqrt_f(float x) { return __builtin_amdgcn_rsqf(x); }

__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += dpp<0x142, 0xa>(v);  // row_bcast 15 into rows 1 and 3
  v += dpp<0x143, 0xc>(v);  // row_bcast 31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x128>(v));
  float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
  float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal: the data is used once).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float fdot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

// Matrix-core product of a 16 x 32 fp16 tile a with a 32 x 16 fp16 tile b, added to
// c.  Lane l supplies a[l % 16][8 (l / 16) + e] and b[8 (l / 16) + e][l % 16] as
// element e of its 8 halves (4 words), and holds c[4 (l / 16) + e][l % 16] as
// element e of its 4 floats (the gfx950 layout of v_mfma_f32_16x16x32_f16).
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4 a, const uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b),
                                                c, 0, 0, 0);
}
// The same product with bf16 operands (same lane layout).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4_t mfma16x16x32_bf16(const uint4 a, const uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// The same product shape with K = 16: lane l supplies a[l % 16][4 (l / 16) + e] and
// b[4 (l / 16) + e][l % 16] as element e of its 4 bf16 (2 words); c as above
// (v_mfma_f32_16x16x16_bf16).
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t mfma16x16x16_bf16(const uint2 a, const uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b),
                                                   c, 0, 0, 0);
}

// (a, b) as bf16 high parts and bf16 low parts (the residuals f - high), packed in pairs;
// round to nearest even (v_cvt_pk_bf16_f32: one instruction per pair).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const uint32_t h = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)a, (__bf16)b});
  const float ra = a - __uint_as_float(h << 16), rb = b - __uint_as_float(h & 0xffff0000u);
  hi = h;
  lo = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)ra, (__bf16)rb});
}

// (a & mask) | bias as one v_and_or_b32.  A three-source VALU instruction takes no
// 32-bit literal on this architecture, so with literal constants the compiler splits
// it into v_and_b32 + v_or_b32.  The empty asm statements only hide the constants'
// values: the mask then lives in a scalar register and the bias in a vector register
// (both set once, outside the loops that use them), and the compiler still emits
// and tracks the instruction itself (its wait states before a matrix-core read of
// the result included).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bias) {
  asm("" : "+s"(mask));
  asm("" : "+v"(bias));
  return (a & mask) | bias;
}

// One 16-byte word group of codes -> the fp16 magic-bias pairs of k_gemv_int4
// (1024 + q for codes in bits 0..3 of a half, 1024 + 16 q for bits 4..7).
__device__ __forceinline__ void dequant16(const uint4 raw, uint32_t (&p)[16]) {
  const uint32_t ww[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t t = ww[q] >> 8;
    p[4 * q + 0] = and_or(ww[q], 0x000F000Fu, 0x64006400u);
    p[4 * q + 1] = and_or(ww[q], 0x00F000F0u, 0x64006400u);
    p[4 * q + 2] = and_or(t, 0x000F000Fu, 0x64006400u);
    p[4 * q + 3] = and_or(t, 0x00F000F0u, 0x64006400u);
  }
}

__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
  half2_t h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

}  // namespace kmr

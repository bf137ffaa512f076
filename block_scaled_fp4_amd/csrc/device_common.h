// device_common.h -- number-format helpers for gfx950 kernels of the FP4 library.
//
// NVFP4 = E2M1 elements with an E4M3 scale per 16 elements (ScaleSearch page,
// Declaracion del Problema).  All helpers here are written for CDNA4: the E2M1
// rounding uses the hardware converter v_cvt_scalef32_pk_fp4_f32 with a unit
// scale (round to nearest even, saturating at 6), the reverse conversion
// v_cvt_scalef32_pk_{f32,f16}_fp4; both apply only the exponent of their scale
// operand, so non power-of-two scales are applied with a separate multiply.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4dev {

typedef _Float16 half_t;
typedef half_t half2_t __attribute__((ext_vector_type(2)));
typedef half_t half4_t __attribute__((ext_vector_type(4)));
typedef half_t half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef uint32_t uint2_t __attribute__((ext_vector_type(2)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));
typedef double double2_t __attribute__((ext_vector_type(2)));

// E4M3 byte (0..0x7E) -> binary32 value, from the field layout: exponent field
// e (bias 7) and 3-bit mantissa m; e = 0 is subnormal m * 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  if (b < 8u) return (float)b * 0x1p-9f;
  return __uint_as_float((((b >> 3) + 120u) << 23) | ((b & 7u) << 20));
}

// Nearest E4M3 byte to v >= +0, ties to the even mantissa, saturating at
// 0x7E = 448 (never the NaN byte 0x7F).  gfx950's fp8 convert rounds to
// nearest even into the OCP E4M3 format, subnormals included, and agrees with
// that rounding on every binary32 in [0, 464]; past 464 it returns the NaN
// code instead of saturating, so the input is first bounded by 448.  The mask
// keeps the byte inside the 128-entry scale tables.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const float b = __builtin_fminf(v, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(b, 0.0f, 0, false) & 0x7Fu;
}

// Nearest E4M3 byte to the exact quotient a/6 (a >= 0 finite).  Exactly the
// E4M3 rounding of the correctly rounded binary32 a/6: binary32 rounding can
// not land on an E4M3 midpoint unless the quotient is that midpoint.  Computed
// without a division: an estimate, then exact comparisons of a with 6 * the
// neighbouring midpoints (6 * midpoint is exact in binary32).
__device__ __forceinline__ uint32_t e4m3_of_div6(float a) {
  uint32_t b = f32_to_e4m3(a * (1.0f / 6.0f));
  float s = e4m3_to_f32(b);
  if (b < 0x7Eu) {
    float up = e4m3_to_f32(b + 1u);
    float mid6 = (s + up) * 3.0f;  // 6 * (s + up) / 2, exact
    if (a > mid6 || (a == mid6 && (b & 1u))) ++b;
  }
  if (b > 0u) {
    float lo = e4m3_to_f32(b - 1u);
    float s2 = e4m3_to_f32(b);
    float mid6 = (lo + s2) * 3.0f;
    if (a < mid6 || (a == mid6 && (b & 1u))) --b;
  }
  return b;
}

// Correctly rounded binary32 a / 6 for normal a (three operations: a product
// with the rounded reciprocal, the exact remainder by a fused multiply-add, one
// fused correction).  Checked against IEEE division for every binary32 in
// 22 binades on the host (the check is in the CPU test suite).
__device__ __forceinline__ float div6_rn(float a) {
  const float r = 1.0f / 6.0f;
  const float q1 = a * r;
  const float rem = __builtin_fmaf(-q1, 6.0f, a);
  return __builtin_fmaf(rem, r, q1);
}

// Two binary32 values t0, t1 >= 0 -> byte (code(t1) << 4) | code(t0) written
// into byte `sel` of `old`; codes are nearest E2M1 (ties to even), saturating.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_pk_fp4(uint32_t old, float t0, float t1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, t0, t1, 1.0f, SEL);
}

// Byte `sel` of src (two E2M1 codes) -> two binary32 values (low nibble first).
template <int SEL>
__device__ __forceinline__ float2_t cvt_pk_f32_fp4(uint32_t src) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(src, 1.0f, SEL);
}

// Byte `sel` of src (two E2M1 codes) -> two fp16 values (low nibble first).
template <int SEL>
__device__ __forceinline__ half2_t cvt_pk_f16_fp4(uint32_t src) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(src, 1.0f, SEL);
}

// bf16 / fp16 / fp32 element loads converted exactly to binary32.
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Correctly rounded binary32 quotient n / d for finite positive n, d, computed
// once per launch or per block: a binary64 estimate and an exact residual check
// of the neighbouring binary32 values.
__device__ __forceinline__ float div_rn(float n, float d) {
  float q = (float)((double)n / (double)d);
  float best = q;
  double bestErr = fabs((double)n - (double)q * (double)d);
  // neighbours of a positive finite binary32 value: adjacent bit patterns
  float cand[2] = {__uint_as_float(__float_as_uint(q) - 1u), __uint_as_float(__float_as_uint(q) + 1u)};
  for (int i = 0; i < 2; ++i) {
    double err = fabs((double)n - (double)cand[i] * (double)d);
    if (err < bestErr) { bestErr = err; best = cand[i]; }
  }
  return best;
}

// Quad-permute a lane value with its neighbour (lane ^ 1) via DPP.
__device__ __forceinline__ float swap_lane1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t swap_lane1_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

// Raw buffer resource over [base, base + bytes): loads through it take a
// 32-bit byte offset and return zero when the access lies past the end, so
// tile loads need neither bounds branches nor 64-bit address arithmetic.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4_t buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint2_t buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load2(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load1(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

}  // namespace fp4dev

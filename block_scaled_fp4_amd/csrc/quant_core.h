// quant_core.h -- the NVFP4 block quantizer shared by the quantize kernels
// and the KV-cache append kernel (ScaleSearch page, Metodologia /
// ScaleSearch): max-scaling start (amax/6 rounded to E4M3), integer offsets on
// the scale byte, least squared error wins.
#pragma once
#include "device_common.h"

namespace fp4dev {

// Scale and reciprocal of every scale byte: {s, fl32(1/s)} with the
// reciprocal correctly rounded (the compiler evaluates 1.0f / s exactly under
// IEEE rules at compile time).  Byte 0 maps to {0, 0}: every element then
// rounds to code 0 and its error is the element itself; byte 0x7F (NaN) is
// never a candidate.
struct ScaleTable {
  float2_t v[128];
  constexpr ScaleTable() : v() {
    for (int b = 0; b < 128; ++b) {
      float s = 0.0f;
      if (b < 8) s = (float)b / 512.0f;
      else {
        int e = (b >> 3) - 7, m = b & 7;
        s = 1.0f + (float)m / 8.0f;
        for (int i = 0; i < e; ++i) s *= 2.0f;
        for (int i = 0; i > e; --i) s /= 2.0f;
      }
      v[b] = (b == 0 || b == 127) ? float2_t{0.0f, 0.0f} : float2_t{s, 1.0f / s};
    }
  }
};
static __constant__ ScaleTable kScaleTab = ScaleTable();

template <typename T>
__device__ __forceinline__ float load_elem(const T* p);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <>
__device__ __forceinline__ float load_elem<half_t>(const half_t* p) { return (float)*p; }
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }

// Load 8 consecutive elements (16-byte aligned for 2-byte types) as binary32.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* y);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* y) {
  uint4_t w = *reinterpret_cast<const uint4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = __uint_as_float(w[i] << 16);
    y[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void load8<half_t>(const half_t* p, float* y) {
  half8_t w = *reinterpret_cast<const half8_t*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (float)w[i];
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* y) {
  float4_t a = *reinterpret_cast<const float4_t*>(p);
  float4_t b = *reinterpret_cast<const float4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { y[i] = a[i]; y[4 + i] = b[i]; }
}

// 8 values -> 8 E2M1 codes in one dword (nearest, ties to the even code,
// saturating at 6; the magnitude is rounded, the sign follows the value).
__device__ __forceinline__ uint32_t pack8(const float* t) {
  // every byte of w is written below: its start value only lends a register
  // (t[0]'s, dead once its pair is converted in the callers)
  uint32_t w = __float_as_uint(t[0]);
  w = cvt_pk_fp4<0>(w, t[0], t[1]);
  w = cvt_pk_fp4<1>(w, t[2], t[3]);
  w = cvt_pk_fp4<2>(w, t[4], t[5]);
  w = cvt_pk_fp4<3>(w, t[6], t[7]);
  return w;
}

// E2M1 values of the 8 codes in a dword.
__device__ __forceinline__ void unpack8(uint32_t w, float* v) {
  float2_t a = cvt_pk_f32_fp4<0>(w), b = cvt_pk_f32_fp4<1>(w);
  float2_t c = cvt_pk_f32_fp4<2>(w), d = cvt_pk_f32_fp4<3>(w);
  v[0] = a[0]; v[1] = a[1]; v[2] = b[0]; v[3] = b[1];
  v[4] = c[0]; v[5] = c[1]; v[6] = d[0]; v[7] = d[1];
}

// Squared error of one 16-element block y for the scale {s, r}.  Values
// keep their sign throughout: y - v*s has the magnitude of |y| - |v|*s (v has
// the sign of y, or is zero), so the squares are those of the definition.
// The sum follows the fixed pairwise tree (0+1, 2+3, ..., then pairs of
// pairs); the product v*s is exact, so fmaf rounds once, like the plain
// difference.
__device__ __forceinline__ float block_sse(const float (&y)[16], float2_t sr) {
  float t[16], v[16], q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = y[i] * sr[1];
  unpack8(pack8(t), v);
  unpack8(pack8(t + 8), v + 8);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float e = __builtin_fmaf(-v[i], sr[0], y[i]);
    q[i] = e * e;
  }
  float l1[8], l2[4];
#pragma unroll
  for (int k = 0; k < 8; ++k) l1[k] = q[2 * k] + q[2 * k + 1];
#pragma unroll
  for (int k = 0; k < 4; ++k) l2[k] = l1[2 * k] + l1[2 * k + 1];
  return (l2[0] + l2[1]) + (l2[2] + l2[3]);
}

// Codes of one block for the reciprocal r (two dwords, element 2i in the low nibble).
__device__ __forceinline__ void block_codes(const float (&y)[16], float r, uint32_t (&c)[2]) {
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = y[i] * r;
  c[0] = pack8(t);
  c[1] = pack8(t + 8);
}

// Sign bits of 16 values at bit 3 of each nibble (two dwords).
__device__ __forceinline__ void sign_nibbles(const float (&y)[16], uint32_t (&m)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= (__float_as_uint(y[8 * h + i]) >> 31) << (4 * i + 3);
    m[h] = w;
  }
}

// One candidate of the offset search: a byte outside 0..0x7E is evaluated on
// byte 0 and can never win.  The comparison runs on the error's bit pattern
// (non-negative floats order like their bits) against a running best that
// starts above every float, so the first valid candidate wins even with an
// infinite error, and later ones only when strictly smaller: ties keep the
// lowest offset.
__device__ __forceinline__ void try_offset(const float (&y)[16], int s0, int f, const float2_t* tab,
                                           uint32_t& best, int& bestf) {
  const int b = s0 + f;
  const bool valid = (unsigned)b <= 0x7Eu;
  const float sse = block_sse(y, tab[valid ? b : 0]);
  const uint32_t key = valid ? __float_as_uint(sse) : 0xFFFFFFFFu;
  const bool better = key < best;
  best = better ? key : best;
  bestf = better ? f : bestf;
}

// Quantize one block of 16 scaled values.  Returns the scale byte, the offset
// and the codes (two dwords, element 2i in the low nibble).  The default
// search range [-2, 6] is fully unrolled; other ranges loop.
__device__ __forceinline__ void quantize_block(const float (&y)[16], int search, int fmin, int fmax,
                                               const float2_t* tab, uint32_t (&codes)[2], uint32_t& scale,
                                               int& off) {
  // a = max |y|; a non-finite element makes the maximum of the magnitude bits
  // reach the exponent-all-ones range
  uint32_t abits = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) abits = __builtin_elementwise_max(abits, __float_as_uint(y[i]) & 0x7FFFFFFFu);
  uint32_t sgn[2];
  sign_nibbles(y, sgn);
  if (abits >= 0x7F800000u || abits == 0u) {
    codes[0] = sgn[0];
    codes[1] = sgn[1];
    scale = abits ? 0x7Fu : 0u;
    off = 0;
    return;
  }
  const int s0 = (int)e4m3_of_div6(__uint_as_float(abits));
  uint32_t best = 0xFFFFFFFFu;
  int bestf = 0;
  if (search && fmin == -2 && fmax == 6) {
#pragma unroll
    for (int f = -2; f <= 6; ++f) try_offset(y, s0, f, tab, best, bestf);
  } else if (search) {
    for (int f = fmin; f <= fmax; ++f) try_offset(y, s0, f, tab, best, bestf);
  }
  // (without the search the only candidate, s0 itself, is always valid)
  scale = (uint32_t)(s0 + bestf);
  off = bestf;
  block_codes(y, tab[scale][1], codes);
  codes[0] |= sgn[0];
  codes[1] |= sgn[1];
}

}  // namespace fp4dev

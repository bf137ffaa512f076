// quantize.hip -- NVFP4 block quantizer with ScaleSearch for gfx950.
//
// ScaleSearch page, Metodologia / ScaleSearch: the block scale starts from
// max-scaling (amax/6 rounded to E4M3); ScaleSearch adds an integer offset f to
// the scale's byte for f in a small range and keeps the scale with the least
// squared error.
//
// The kernel is VALU-bound with the search on (9 candidates x 16 elements per
// block), HBM-bound without it.  Layout choices:
//   block_axis 0 (blocks along the contiguous dimension): two lanes share a
//     block, 8 elements each, so one 16-byte load per lane covers a bf16 block
//     half and a wavefront reads 2 KiB of contiguous input; the partial error
//     sums of the two lanes meet through a DPP quad permute.
//   block_axis 1 (blocks along rows, e.g. V along tokens): one lane per block,
//     consecutive lanes take consecutive columns, so each of the 16 row loads
//     of a wavefront is one contiguous 128-byte (bf16) segment.
// Error sums follow one fixed pairwise tree ((0+1),(2+3),... then pairs of
// pairs), element errors are |y| - v*s with an exact product, and nothing is
// contracted, so the chosen offsets are the same on every run and platform.
#include "device_common.h"
#include "fp4_internal.h"

namespace fp4dev {

// Reciprocals of every scale byte, correctly rounded binary32, built at
// compile time (the compiler evaluates 1.0f / s exactly under IEEE rules).
struct RecipTable {
  float v[128];
  constexpr RecipTable() : v() {
    for (int b = 0; b < 128; ++b) {
      float s = 0.0f;
      if (b < 8) s = (float)b / 512.0f;
      else {
        int e = (b >> 3) - 7, m = b & 7;
        s = 1.0f + (float)m / 8.0f;
        for (int i = 0; i < e; ++i) s *= 2.0f;
        for (int i = 0; i > e; --i) s /= 2.0f;
      }
      v[b] = (b == 0 || b == 127) ? 0.0f : 1.0f / s;
    }
  }
};
__constant__ RecipTable kRecip = RecipTable();

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
__device__ __forceinline__ void load8(const T* p, float (&y)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&y)[8]) {
  uint4_t w = *reinterpret_cast<const uint4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = __uint_as_float(w[i] << 16);
    y[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void load8<half_t>(const half_t* p, float (&y)[8]) {
  half8_t w = *reinterpret_cast<const half8_t*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (float)w[i];
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&y)[8]) {
  float4_t a = *reinterpret_cast<const float4_t*>(p);
  float4_t b = *reinterpret_cast<const float4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { y[i] = a[i]; y[4 + i] = b[i]; }
}

// Convert 8 non-negative values to 8 E2M1 codes packed in one dword.
__device__ __forceinline__ uint32_t pack8(const float (&t)[8]) {
  uint32_t w = 0;
  w = cvt_pk_fp4<0>(w, t[0], t[1]);
  w = cvt_pk_fp4<1>(w, t[2], t[3]);
  w = cvt_pk_fp4<2>(w, t[4], t[5]);
  w = cvt_pk_fp4<3>(w, t[6], t[7]);
  return w;
}

// E2M1 values of the 8 codes in a dword.
__device__ __forceinline__ void unpack8(uint32_t w, float (&v)[8]) {
  float2_t a = cvt_pk_f32_fp4<0>(w), b = cvt_pk_f32_fp4<1>(w);
  float2_t c = cvt_pk_f32_fp4<2>(w), d = cvt_pk_f32_fp4<3>(w);
  v[0] = a[0]; v[1] = a[1]; v[2] = b[0]; v[3] = b[1];
  v[4] = c[0]; v[5] = c[1]; v[6] = d[0]; v[7] = d[1];
}

// Sum of 8 squared errors by the fixed pairwise tree (elements 0..7 of a half block).
__device__ __forceinline__ float tree8(const float (&q)[8]) {
  float a0 = q[0] + q[1], a1 = q[2] + q[3], a2 = q[4] + q[5], a3 = q[6] + q[7];
  float b0 = a0 + a1, b1 = a2 + a3;
  return b0 + b1;
}

// Squared error of 8 elements |y| for scale byte b (b > 0), and their codes.
__device__ __forceinline__ float half_block_sse(const float (&ay)[8], uint32_t b, const float* recip,
                                                uint32_t& codes) {
  float s = e4m3_to_f32(b);
  float r = recip[b];
  float t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = ay[i] * r;
  codes = pack8(t);
  float v[8], q[8];
  unpack8(codes, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float e = __builtin_fmaf(-v[i], s, ay[i]);  // |y| - v*s: the product is exact, one rounding
    q[i] = e * e;
  }
  return tree8(q);
}

__device__ __forceinline__ float half_block_sse_zero(const float (&ay)[8]) {
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = ay[i] * ay[i];
  return tree8(q);
}

// Sign bits of 8 elements placed at bit 3 of each nibble.
__device__ __forceinline__ uint32_t sign_nibbles(const float (&y)[8]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m |= (__float_as_uint(y[i]) >> 31) << (4 * i + 3);
  return m;
}

// Choose the scale of one block held as NH halves of 8 elements per lane
// (NH = 1: the other half is on lane ^ 1; NH = 2: the whole block on this lane).
// Returns the scale byte, the offset and the packed codes (one dword per half).
template <int NH>
__device__ __forceinline__ void choose_block(const float (&y)[NH][8], int search, int fmin, int fmax,
                                             const float* recip, uint32_t (&codes)[NH],
                                             uint32_t& scale, int& off) {
  float ay[NH][8];
  float a = 0.0f;
  bool bad = false;
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ay[h][i] = __builtin_fabsf(y[h][i]);
      bad |= !__builtin_isfinite(y[h][i]);
      a = __builtin_fmaxf(a, ay[h][i]);
    }
  if (NH == 1) {
    a = __builtin_fmaxf(a, swap_lane1(a));
    bad |= swap_lane1_u((uint32_t)bad) != 0u;
  }
  uint32_t sgn[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) sgn[h] = sign_nibbles(y[h]);
  if (bad || a == 0.0f) {
#pragma unroll
    for (int h = 0; h < NH; ++h) codes[h] = sgn[h];
    scale = bad ? 0x7Fu : 0u;
    off = 0;
    return;
  }
  const int s0 = (int)e4m3_of_div6(a);
  const int lo = search ? fmin : 0, hi = search ? fmax : 0;
  // Branch-free candidate loop (the bounds are uniform): a byte outside
  // 0..0x7E is evaluated on a clamped byte and given an infinite error; byte 0
  // needs no special case because its reciprocal entry is 0, which maps every
  // element to code 0 and leaves the error |y| itself.
  float best = 0.0f;
  bool have = false;  // a valid candidate has been seen (the first one always wins, even at inf)
  int bestf = 0;
  uint32_t bestc[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) bestc[h] = 0;
#pragma unroll 3
  for (int f = lo; f <= hi; ++f) {
    const int b = s0 + f;
    const bool valid = b >= 0 && b <= 0x7E;
    const uint32_t bc = (uint32_t)(b < 0 ? 0 : (b > 0x7E ? 0x7E : b));
    float part[NH];
    uint32_t c[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) part[h] = half_block_sse(ay[h], bc, recip, c[h]);
    float sse;
    if (NH == 1) {
      float other = swap_lane1(part[0]);
      sse = part[0] + other;  // elements 0..7 tree + elements 8..15 tree (commutative)
    } else {
      sse = part[0] + part[NH - 1];
    }
    const bool better = valid && (!have || sse < best);
    have = have || valid;
    if (better) {
      best = sse;
      bestf = f;
#pragma unroll
      for (int h = 0; h < NH; ++h) bestc[h] = c[h];
    }
  }
#pragma unroll
  for (int h = 0; h < NH; ++h) codes[h] = bestc[h] | sgn[h];
  scale = (uint32_t)(s0 + bestf);
  off = bestf;
}

struct QuantArgs {
  const void* x;
  int64_t rows, cols, ld;
  uint32_t* codes;  // axis 0: as dwords; axis 1: bytes via codes8
  uint8_t* codes8;
  uint8_t* scales;
  int8_t* offsets;
  float* g;          // per-tensor scale output/input (may be null for mode 0)
  const float* amax_part;  // partial maxima (mode 1)
  int n_part;
  int search, fmin, fmax, gmode;
};

// Per-tensor scale factors from the partial maxima (mode 1) or *g (mode 2).
// Every thread of the workgroup reads at most a few partials; the maximum is
// reduced through LDS, then thread 0 forms the correctly rounded factors.
__device__ __forceinline__ void global_factors(const QuantArgs& A, float* sh, float& ginv) {
  if (A.gmode == 0) { ginv = 1.0f; return; }
  float a = 0.0f;
  if (A.gmode == 1)
    for (int i = threadIdx.x; i < A.n_part; i += blockDim.x) a = __builtin_fmaxf(a, A.amax_part[i]);
  sh[threadIdx.x] = a;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] = __builtin_fmaxf(sh[threadIdx.x], sh[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float gi = 1.0f, g = 1.0f;
    if (A.gmode == 2) {
      g = *A.g;
      gi = div_rn(1.0f, g);
    } else {
      a = sh[0];
      if (a > 0.0f && __builtin_isfinite(a)) {
        g = div_rn(a, 2688.0f);
        gi = div_rn(2688.0f, a);
      } else if (a > 0.0f) {  // infinite amax: g = inf, every finite element scales to 0
        g = __builtin_inff();
        gi = 0.0f;
      }
      if (blockIdx.x == 0) *A.g = g;
    }
    sh[256] = gi;
  }
  __syncthreads();
  ginv = sh[256];
}

// block_axis 0: 2 lanes per 16-element block.
template <typename T>
__global__ void __launch_bounds__(256) quantize_axis0_kernel(QuantArgs A) {
  __shared__ float recip[128];
  __shared__ float sh[257];
  if (threadIdx.x < 128) recip[threadIdx.x] = kRecip.v[threadIdx.x];
  float ginv;
  global_factors(A, sh, ginv);
  __syncthreads();
  const int64_t bpr = A.cols / 16;  // blocks per row
  const int64_t nhalf = A.rows * bpr * 2;
  const T* x = reinterpret_cast<const T*>(A.x);
  for (int64_t hi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; hi - (threadIdx.x & 1) < nhalf;
       hi += (int64_t)gridDim.x * blockDim.x) {
    // both lanes of a pair stay in the loop together (nhalf is even)
    const int64_t blk = hi >> 1;
    const int64_t r = blk / bpr, cb = blk - r * bpr;
    const int part = (int)(hi & 1);
    float y[1][8];
    load8<T>(x + r * A.ld + cb * 16 + part * 8, y[0]);
    if (A.gmode != 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[0][i] = y[0][i] * ginv;
    }
    uint32_t codes[1], scale;
    int off;
    choose_block<1>(y, A.search, A.fmin, A.fmax, recip, codes, scale, off);
    A.codes[hi] = codes[0];
    if (part == 0) {
      A.scales[blk] = (uint8_t)scale;
      if (A.offsets) A.offsets[blk] = (int8_t)off;
    }
  }
}

// block_axis 1: one lane per block of 16 rows of one column.
template <typename T>
__global__ void __launch_bounds__(256) quantize_axis1_kernel(QuantArgs A) {
  __shared__ float recip[128];
  __shared__ float sh[257];
  if (threadIdx.x < 128) recip[threadIdx.x] = kRecip.v[threadIdx.x];
  float ginv;
  global_factors(A, sh, ginv);
  __syncthreads();
  const int64_t nb = (A.rows / 16) * A.cols;
  const T* x = reinterpret_cast<const T*>(A.x);
  for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < nb;
       blk += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rb = blk / A.cols, c = blk - rb * A.cols;
    float y[2][8];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float v = load_elem<T>(x + (rb * 16 + k) * A.ld + c);
      y[k >> 3][k & 7] = A.gmode != 0 ? v * ginv : v;
    }
    uint32_t codes[2], scale;
    int off;
    choose_block<2>(y, A.search, A.fmin, A.fmax, recip, codes, scale, off);
    // row pair (2i, 2i+1) -> byte i of the block's 8 bytes, at codes8[(rb*8+i)*cols + c]
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t byte = (codes[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      A.codes8[(rb * 8 + i) * A.cols + c] = (uint8_t)byte;
    }
    A.scales[blk] = (uint8_t)scale;
    if (A.offsets) A.offsets[blk] = (int8_t)off;
  }
}

// Partial maxima of |x| (NaN ignored) for the per-tensor scale: one per
// workgroup, grid-stride over rows with 8-element (16-byte for 2-byte types)
// loads when rows are dense.
template <typename T>
__global__ void __launch_bounds__(256) amax_kernel(const T* x, int64_t rows, int64_t cols, int64_t ld,
                                                   float* part) {
  __shared__ float red[256];
  float m = 0.0f;
  if (cols % 8 == 0 && ld % 8 == 0) {
    const int64_t per_row = cols / 8, n = rows * per_row;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
      const int64_t r = i / per_row, c = (i - r * per_row) * 8;
      float y[8];
      load8<T>(x + r * ld + c, y);
#pragma unroll
      for (int k = 0; k < 8; ++k) m = __builtin_fmaxf(m, __builtin_fabsf(y[k]));
    }
  } else {
    const int64_t n = rows * cols;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
      int64_t r = i / cols, c = i - r * cols;
      m = __builtin_fmaxf(m, __builtin_fabsf(load_elem<T>(x + r * ld + c)));
    }
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = __builtin_fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

__global__ void set_one_kernel(float* g) { *g = 1.0f; }

}  // namespace fp4dev

using namespace fp4dev;

int fp4i_amax_parts(int64_t rows, int64_t cols) {
  // enough workgroups to stream the tensor at full bandwidth, few enough that
  // every quantize workgroup can re-reduce them cheaply
  int64_t n = rows * cols;
  int64_t p = (n + 256 * 64 - 1) / (256 * 64);
  if (p < 1) p = 1;
  if (p > 512) p = 512;
  return (int)p;
}

hipError_t fp4i_launch_quantize(const QuantLaunch& L, hipStream_t stream) {
  QuantArgs A;
  A.x = L.x;
  A.rows = L.rows;
  A.cols = L.cols;
  A.ld = L.ld;
  A.codes = reinterpret_cast<uint32_t*>(L.codes);
  A.codes8 = L.codes;
  A.scales = L.scales;
  A.offsets = L.offsets;
  A.g = L.g;
  A.search = L.search;
  A.fmin = L.fmin;
  A.fmax = L.fmax;
  A.gmode = L.gmode;
  A.amax_part = L.amax_ws;
  A.n_part = 0;
  if (L.rows == 0 || L.cols == 0) {
    if (L.g && L.gmode != 2) hipLaunchKernelGGL(set_one_kernel, dim3(1), dim3(1), 0, stream, L.g);
    return hipGetLastError();
  }
  if (L.gmode == 1) {
    A.n_part = fp4i_amax_parts(L.rows, L.cols);
    if (L.dtype == 0)
      hipLaunchKernelGGL(amax_kernel<uint16_t>, dim3(A.n_part), dim3(256), 0, stream,
                         (const uint16_t*)L.x, L.rows, L.cols, L.ld, L.amax_ws);
    else if (L.dtype == 1)
      hipLaunchKernelGGL(amax_kernel<half_t>, dim3(A.n_part), dim3(256), 0, stream,
                         (const half_t*)L.x, L.rows, L.cols, L.ld, L.amax_ws);
    else
      hipLaunchKernelGGL(amax_kernel<float>, dim3(A.n_part), dim3(256), 0, stream,
                         (const float*)L.x, L.rows, L.cols, L.ld, L.amax_ws);
  } else if (L.gmode == 0 && L.g) {
    hipLaunchKernelGGL(set_one_kernel, dim3(1), dim3(1), 0, stream, L.g);
  }
  int64_t work = L.axis == 0 ? L.rows * (L.cols / 16) * 2 : (L.rows / 16) * L.cols;
  int64_t grid = (work + 255) / 256;
  if (grid > 65536) grid = 65536;
  if (grid < 1) grid = 1;
  if (L.axis == 0) {
    if (L.dtype == 0) hipLaunchKernelGGL(quantize_axis0_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream, A);
    else if (L.dtype == 1) hipLaunchKernelGGL(quantize_axis0_kernel<half_t>, dim3(grid), dim3(256), 0, stream, A);
    else hipLaunchKernelGGL(quantize_axis0_kernel<float>, dim3(grid), dim3(256), 0, stream, A);
  } else {
    if (L.dtype == 0) hipLaunchKernelGGL(quantize_axis1_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream, A);
    else if (L.dtype == 1) hipLaunchKernelGGL(quantize_axis1_kernel<half_t>, dim3(grid), dim3(256), 0, stream, A);
    else hipLaunchKernelGGL(quantize_axis1_kernel<float>, dim3(grid), dim3(256), 0, stream, A);
  }
  return hipGetLastError();
}

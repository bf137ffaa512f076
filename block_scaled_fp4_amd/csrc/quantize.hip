// quantize.hip -- NVFP4 block quantizer with ScaleSearch for gfx950.
//
// ScaleSearch page, Metodologia / ScaleSearch: the block scale starts from
// max-scaling (amax/6 rounded to E4M3); ScaleSearch adds an integer offset f to
// the scale's byte for f in a small range and keeps the scale with the least
// squared error.
//
// The kernel is VALU-bound with the search on (9 candidates x 16 elements per
// block), HBM-bound without it.  Layout choices:
//   block_axis 0 (blocks along the contiguous dimension): one lane per block,
//     two 16-byte loads for bf16, so a wavefront reads 2 KiB of contiguous
//     input and writes 512 contiguous code bytes; the default offset range is
//     fully unrolled and each candidate is a straight run of multiplies,
//     hardware E2M1 converts (there and back),
//     fused error terms, squares and the fixed sum tree; the codes of the
//     chosen scale are formed once at the end.
//   block_axis 1 (blocks along rows, e.g. V along tokens): one lane per block,
//     consecutive lanes take consecutive columns, so each of the 16 row loads
//     of a wavefront is one contiguous 128-byte (bf16) segment.
// Error sums follow one fixed pairwise tree ((0+1),(2+3),... then pairs of
// pairs), element errors are |y| - v*s with an exact product, and nothing is
// contracted, so the chosen offsets are the same on every run and platform.
#include "device_common.h"
#include "fp4_internal.h"
#include "quant_core.h"

namespace fp4dev {

struct QuantArgs {
  const void* x;
  int64_t rows, cols, ld;
  uint2_t* codes;   // axis 0: one 8-byte pair of dwords per block
  uint8_t* codes8;  // axis 1: bytes
  uint8_t* scales;
  int8_t* offsets;
  float* g;                // per-tensor scale output/input (may be null for mode 0)
  const float* amax_part;  // partial maxima (mode 1)
  int n_part;
  int search, fmin, fmax, gmode;
  uint32_t hsigns[4];  // incoherence processing: sign bits and 1/sqrt(cols)
  float hscale;
};

// Incoherence processing of one row held by the bpr = cols/16 consecutive
// lanes of its blocks (ScaleSearch page, Metodologia / ScaleSearchAttention):
// signs, then the Hadamard butterflies of span 1, 2, 4, 8 inside the lane and
// 16, 32, 64 across lanes (lane ^ 1, 2, 4), each pair (a, b) -> (a + b, a - b)
// in binary32, then the 1/sqrt(cols) multiply.  All lanes of a row are active
// together (rows are whole in the grid-stride loop).
__device__ __forceinline__ void hadamard_block(float (&y)[16], const QuantArgs& A, int64_t cb, int bpr) {
  const uint32_t sm = (A.hsigns[cb >> 1] >> ((cb & 1) * 16)) & 0xFFFFu;
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = __uint_as_float(__float_as_uint(y[i]) ^ (((sm >> i) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!(i & h)) {
        const float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
  const int lane = threadIdx.x;
  for (int hb = 1; hb < bpr; hb <<= 1) {
    const bool upper = (lane & hb) != 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float o = __shfl_xor(y[i], hb, 64);
      y[i] = upper ? o - y[i] : y[i] + o;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = y[i] * A.hscale;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, k, 64));
  return v;
}

// Per-tensor encode factor from the partial maxima (mode 1) or *g (mode 2):
// every thread reads a few partials, waves reduce with cross-lane moves and
// one LDS exchange joins the waves.  The first workgroup writes g (mode 1).
__device__ __forceinline__ float global_factor(const QuantArgs& A, float* sh) {
  if (A.gmode == 0) return 1.0f;
  if (A.gmode == 2) return div_rn(1.0f, *A.g);
  float a = 0.0f;
  for (int i = threadIdx.x; i < A.n_part; i += blockDim.x) a = __builtin_fmaxf(a, A.amax_part[i]);
  a = wave_max(a);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = a;
  __syncthreads();
  a = sh[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) a = __builtin_fmaxf(a, sh[w]);
  float g = 1.0f, gi = 1.0f;
  if (a > 0.0f && __builtin_isfinite(a)) {
    g = div_rn(a, 2688.0f);
    gi = div_rn(2688.0f, a);
  } else if (a > 0.0f) {  // infinite amax: g = inf, every finite element scales to 0
    g = __builtin_inff();
    gi = 0.0f;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *A.g = g;
  return gi;
}

// One block of 16 consecutive elements as raw 16-byte words (bf16/fp16: 2,
// fp32: 4), loaded ahead of its use.
template <typename T>
struct RawBlock {
  static constexpr int N = sizeof(T) * 16 / 16;
  uint4_t w[N];
};
template <typename T>
__device__ __forceinline__ void load_raw(RawBlock<T>& R, const T* p) {
#pragma unroll
  for (int i = 0; i < RawBlock<T>::N; ++i) R.w[i] = reinterpret_cast<const uint4_t*>(p)[i];
}
template <typename T>
__device__ __forceinline__ void raw_to_f32(const RawBlock<T>& R, float (&y)[16]);
template <>
__device__ __forceinline__ void raw_to_f32<uint16_t>(const RawBlock<uint16_t>& R, float (&y)[16]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = R.w[i >> 2][i & 3];
    y[2 * i] = __uint_as_float(w << 16);
    y[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void raw_to_f32<half_t>(const RawBlock<half_t>& R, float (&y)[16]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = R.w[i >> 2][i & 3];
    const half2_t h = __builtin_bit_cast(half2_t, w);
    y[2 * i] = (float)h[0];
    y[2 * i + 1] = (float)h[1];
  }
}
template <>
__device__ __forceinline__ void raw_to_f32<float>(const RawBlock<float>& R, float (&y)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = __uint_as_float(R.w[i >> 2][i & 3]);
}

// block_axis 0: one lane per 16-element block; a wavefront reads 64
// consecutive blocks (2 KiB of bf16) and writes their 512 code bytes.  The
// grid is a few workgroups per CU that stride over the blocks, each lane
// loading its next block while it searches the current one.
template <typename T, bool HAD>
__global__ void __launch_bounds__(256) quantize_axis0_kernel(QuantArgs A) {
  __shared__ float2_t tab[128];
  __shared__ float sh[8];
  if (threadIdx.x < 128) tab[threadIdx.x] = kScaleTab.v[threadIdx.x];
  const float ginv = global_factor(A, sh);
  __syncthreads();
  const int64_t bpr = A.cols / 16;  // blocks per row
  const int64_t nb = A.rows * bpr;
  const T* x = reinterpret_cast<const T*>(A.x);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  auto src = [&](int64_t blk) {
    const int64_t r = blk / bpr, cb = blk - r * bpr;
    return x + r * A.ld + cb * 16;
  };
  int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  RawBlock<T> raw;
  if (blk < nb) load_raw<T>(raw, src(blk));
  for (; blk < nb; blk += stride) {
    float y[16];
    raw_to_f32<T>(raw, y);
    if (blk + stride < nb) load_raw<T>(raw, src(blk + stride));
    if (HAD) hadamard_block(y, A, blk % bpr, (int)bpr);
    if (A.gmode != 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = y[i] * ginv;
    }
    uint32_t codes[2], scale;
    int off;
    quantize_block(y, A.search, A.fmin, A.fmax, tab, codes, scale, off);
    A.codes[blk] = uint2_t{codes[0], codes[1]};
    A.scales[blk] = (uint8_t)scale;
    if (A.offsets) A.offsets[blk] = (int8_t)off;
  }
}

// block_axis 1: one lane per block of 16 rows of one column; consecutive
// lanes take consecutive columns, so each row load of a wavefront is one
// contiguous segment.
template <typename T>
__global__ void __launch_bounds__(256) quantize_axis1_kernel(QuantArgs A) {
  __shared__ float2_t tab[128];
  __shared__ float sh[8];
  if (threadIdx.x < 128) tab[threadIdx.x] = kScaleTab.v[threadIdx.x];
  const float ginv = global_factor(A, sh);
  __syncthreads();
  const int64_t nb = (A.rows / 16) * A.cols;
  const T* x = reinterpret_cast<const T*>(A.x);
  for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < nb;
       blk += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rb = blk / A.cols, c = blk - rb * A.cols;
    float y[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float v = load_elem<T>(x + (rb * 16 + k) * A.ld + c);
      y[k] = A.gmode != 0 ? v * ginv : v;
    }
    uint32_t codes[2], scale;
    int off;
    quantize_block(y, A.search, A.fmin, A.fmax, tab, codes, scale, off);
    // row pair (2i, 2i+1) -> byte i of the block's 8 bytes, at codes8[(rb*8+i)*cols + c]
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t byte = (codes[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      A.codes8[(rb * 8 + i) * A.cols + c] = (uint8_t)byte;
    }
    A.scales[blk] = (uint8_t)scale;
    if (A.offsets) A.offsets[blk] = (int8_t)off;
  }
}

// Partial maxima of |x| (NaN ignored) for the per-tensor scale: one per
// workgroup.  Dense rows are read as 16-byte chunks, four per thread in flight.
template <typename T>
__global__ void __launch_bounds__(256) amax_kernel(const T* x, int64_t rows, int64_t cols, int64_t ld,
                                                   float* part) {
  __shared__ float red[4];
  float m = 0.0f;
  if (cols % 8 == 0 && ld % 8 == 0) {
    const int64_t per_row = cols / 8, n = rows * per_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
      float y[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t j = i + u * stride, r = j / per_row, c = (j - r * per_row) * 8;
        load8<T>(x + r * ld + c, y[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) m = __builtin_fmaxf(m, __builtin_fabsf(y[u][k]));
    }
    for (; i < n; i += stride) {
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
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    part[blockIdx.x] = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
}

__global__ void set_one_kernel(float* g) { *g = 1.0f; }

// ---- MXFP4: E2M1 elements, one power-of-two (E8M0) scale per 32 ----------
// (the block floating point the ScaleSearch page contrasts NVFP4 with,
// Declaracion del Problema), scale rule of the OCP microscaling format:
// shared exponent floor(log2(amax)) - 2, clamped to [-127, 127], elements
// RNE-rounded to E2M1 with saturation at 6 (so [6, 8) x scale clips to 6).

struct MxArgs {
  const void* x;
  int64_t rows, cols, ld;
  uint8_t* codes;
  uint8_t* scales;
};

// 32 values -> 16 code bytes (4 dwords, element 2i in the low nibble) and the
// scale byte.
__device__ __forceinline__ void mx_block(const float (&y)[32], uint32_t (&c)[4], uint32_t& sb) {
  uint32_t abits = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) abits = __builtin_elementwise_max(abits, __float_as_uint(y[i]) & 0x7FFFFFFFu);
  uint32_t sgn[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) sgn[i >> 3] |= (__float_as_uint(y[i]) >> 31) << (4 * (i & 7) + 3);
  if (abits >= 0x7F800000u) {  // Inf or NaN in the block
    sb = 0xFFu;
#pragma unroll
    for (int w = 0; w < 4; ++w) c[w] = 0u;
    return;
  }
  int shared = -127;
  if (abits) {
    shared = __builtin_amdgcn_frexp_expf(__uint_as_float(abits)) - 3;  // floor(log2 a) - 2
    shared = shared < -127 ? -127 : (shared > 127 ? 127 : shared);
  }
  sb = (uint32_t)(shared + 127);
  float t[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) t[i] = __builtin_ldexpf(__builtin_fabsf(y[i]), -shared);  // exact: power of two
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t v = 0;
    v = cvt_pk_fp4<0>(v, t[8 * w + 0], t[8 * w + 1]);
    v = cvt_pk_fp4<1>(v, t[8 * w + 2], t[8 * w + 3]);
    v = cvt_pk_fp4<2>(v, t[8 * w + 4], t[8 * w + 5]);
    v = cvt_pk_fp4<3>(v, t[8 * w + 6], t[8 * w + 7]);
    c[w] = v | sgn[w];
  }
}

// One lane per block of 32 consecutive elements of a row.
template <typename T>
__global__ void __launch_bounds__(256) mx_quantize_axis0_kernel(MxArgs A) {
  const int64_t bpr = A.cols / 32;
  const int64_t nb = A.rows * bpr;
  const T* x = reinterpret_cast<const T*>(A.x);
  for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < nb; blk += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = blk / bpr, cb = blk - r * bpr;
    const T* src = x + r * A.ld + cb * 32;
    float y[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) load8<T>(src + 8 * i, y + 8 * i);
    uint32_t c[4], sb;
    mx_block(y, c, sb);
    *reinterpret_cast<uint4_t*>(A.codes + r * (A.cols / 2) + cb * 16) = uint4_t{c[0], c[1], c[2], c[3]};
    A.scales[blk] = (uint8_t)sb;
  }
}

// One lane per block of 32 rows of one column (consecutive lanes, consecutive
// columns).
template <typename T>
__global__ void __launch_bounds__(256) mx_quantize_axis1_kernel(MxArgs A) {
  const int64_t nb = (A.rows / 32) * A.cols;
  const T* x = reinterpret_cast<const T*>(A.x);
  for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < nb; blk += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rb = blk / A.cols, c = blk - rb * A.cols;
    float y[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) y[k] = load_elem<T>(x + (rb * 32 + k) * A.ld + c);
    uint32_t cw[4], sb;
    mx_block(y, cw, sb);
    // row pair (2i, 2i+1) -> byte i of the block's 16 bytes, at codes[(rb*16 + i)*cols + c]
#pragma unroll
    for (int i = 0; i < 16; ++i)
      A.codes[(rb * 16 + i) * A.cols + c] = (uint8_t)((cw[i >> 2] >> (8 * (i & 3))) & 0xFFu);
    A.scales[blk] = (uint8_t)sb;
  }
}

}  // namespace fp4dev

using namespace fp4dev;

int fp4i_amax_parts(int64_t rows, int64_t cols) {
  // enough workgroups to stream the tensor at full bandwidth, few enough that
  // every quantize workgroup can re-reduce them cheaply
  int64_t n = rows * cols;
  int64_t p = (n + 256 * 32 - 1) / (256 * 32);
  if (p < 1) p = 1;
  if (p > 1024) p = 1024;
  return (int)p;
}

hipError_t fp4i_launch_quantize(const QuantLaunch& L, hipStream_t stream) {
  QuantArgs A;
  A.x = L.x;
  A.rows = L.rows;
  A.cols = L.cols;
  A.ld = L.ld;
  A.codes = reinterpret_cast<uint2_t*>(L.codes);
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
  int64_t work = L.axis == 0 ? L.rows * (L.cols / 16) : (L.rows / 16) * L.cols;
  int64_t grid = (work + 255) / 256;
  if (grid > 2048) grid = 2048;  // 8 workgroups per CU, striding over the blocks
  if (grid < 1) grid = 1;
  for (int i = 0; i < 4; ++i) A.hsigns[i] = L.hsigns[i];
  A.hscale = L.hscale;
  if (L.axis == 0 && L.hadamard) {
    if (L.dtype == 0) hipLaunchKernelGGL((quantize_axis0_kernel<uint16_t, true>), dim3(grid), dim3(256), 0, stream, A);
    else if (L.dtype == 1) hipLaunchKernelGGL((quantize_axis0_kernel<half_t, true>), dim3(grid), dim3(256), 0, stream, A);
    else hipLaunchKernelGGL((quantize_axis0_kernel<float, true>), dim3(grid), dim3(256), 0, stream, A);
  } else if (L.axis == 0) {
    if (L.dtype == 0) hipLaunchKernelGGL((quantize_axis0_kernel<uint16_t, false>), dim3(grid), dim3(256), 0, stream, A);
    else if (L.dtype == 1) hipLaunchKernelGGL((quantize_axis0_kernel<half_t, false>), dim3(grid), dim3(256), 0, stream, A);
    else hipLaunchKernelGGL((quantize_axis0_kernel<float, false>), dim3(grid), dim3(256), 0, stream, A);
  } else {
    if (L.dtype == 0) hipLaunchKernelGGL(quantize_axis1_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream, A);
    else if (L.dtype == 1) hipLaunchKernelGGL(quantize_axis1_kernel<half_t>, dim3(grid), dim3(256), 0, stream, A);
    else hipLaunchKernelGGL(quantize_axis1_kernel<float>, dim3(grid), dim3(256), 0, stream, A);
  }
  return hipGetLastError();
}

hipError_t fp4i_launch_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int axis,
                                   uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  MxArgs A;
  A.x = x; A.rows = rows; A.cols = cols; A.ld = ld; A.codes = codes; A.scales = scales;
  const int64_t work = axis == 0 ? rows * (cols / 32) : (rows / 32) * cols;
  if (work == 0) return hipSuccess;
  int64_t grid = (work + 255) / 256;
  if (grid > 2048) grid = 2048;
  if (axis == 0) {
    if (dtype == 0) hipLaunchKernelGGL(mx_quantize_axis0_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream, A);
    else if (dtype == 1) hipLaunchKernelGGL(mx_quantize_axis0_kernel<half_t>, dim3(grid), dim3(256), 0, stream, A);
    else hipLaunchKernelGGL(mx_quantize_axis0_kernel<float>, dim3(grid), dim3(256), 0, stream, A);
  } else {
    if (dtype == 0) hipLaunchKernelGGL(mx_quantize_axis1_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream, A);
    else if (dtype == 1) hipLaunchKernelGGL(mx_quantize_axis1_kernel<half_t>, dim3(grid), dim3(256), 0, stream, A);
    else hipLaunchKernelGGL(mx_quantize_axis1_kernel<float>, dim3(grid), dim3(256), 0, stream, A);
  }
  return hipGetLastError();
}

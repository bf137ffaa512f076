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
  const int32_t* cexp;  // balance exponents [rows / exp_rows][cols] (BAL instances)
  int exp_negate;
  int64_t exp_rows;
  double* means;  // block means of the input (quantize_means_kernel): [rows / mS][mnb][cols]
  int64_t mS;     // rows per head
  int mblk, mnb;  // rows per selection block, blocks per head
  int strided;    // rows at map.row_off(r) (attention inputs with strides), else r * ld
  TokMap map;
  __device__ __forceinline__ int64_t row_off(int64_t r) const { return strided ? map.row_off(r) : r * ld; }
  __device__ __forceinline__ int64_t row_step() const { return strided ? map.ts : ld; }
};

// Magnitude balance of one block (ScaleSearch page, Metodologia /
// ScaleSearchAttention, the pair Q' = Q R^-T, K' = K R with R = diag(2^e)):
// element i of block cb of row r times 2^(+-e[r / exp_rows][16 cb + i]),
// exact in binary32 (v_ldexp_f32).
__device__ __forceinline__ void balance_block(float (&y)[16], const QuantArgs& A, int64_t r, int64_t cb) {
  const uint4_t* ep = reinterpret_cast<const uint4_t*>(A.cexp + (r / A.exp_rows) * A.cols + cb * 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4_t w = ep[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = (int)w[i];
      y[4 * j + i] = __builtin_ldexpf(y[4 * j + i], A.exp_negate ? -e : e);
    }
  }
}

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
// The work of workgroup wg of nwg (grid-stride over the blocks), with the
// scale table in LDS and the per-tensor factor ginv.
template <typename T, bool HAD, bool BAL>
__device__ __forceinline__ void axis0_body(const QuantArgs& A, const float2_t* tab, float ginv, int64_t wg,
                                           int64_t nwg) {
  const int64_t bpr = A.cols / 16;  // blocks per row
  const int64_t nb = A.rows * bpr;
  const T* x = reinterpret_cast<const T*>(A.x);
  const int64_t stride = nwg * blockDim.x;
  auto src = [&](int64_t blk) {
    const int64_t r = blk / bpr, cb = blk - r * bpr;
    return x + A.row_off(r) + cb * 16;
  };
  int64_t blk = wg * blockDim.x + threadIdx.x;
  RawBlock<T> raw;
  if (blk < nb) load_raw<T>(raw, src(blk));
  for (; blk < nb; blk += stride) {
    float y[16];
    raw_to_f32<T>(raw, y);
    if (blk + stride < nb) load_raw<T>(raw, src(blk + stride));
    if (BAL) balance_block(y, A, blk / bpr, blk % bpr);
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

template <typename T, bool HAD, bool BAL>
__global__ void __launch_bounds__(256) quantize_axis0_kernel(QuantArgs A) {
  __shared__ float2_t tab[128];
  __shared__ float sh[8];
  if (threadIdx.x < 128) tab[threadIdx.x] = kScaleTab.v[threadIdx.x];
  const float ginv = global_factor(A, sh);
  __syncthreads();
  axis0_body<T, HAD, BAL>(A, tab, ginv, blockIdx.x, gridDim.x);
}

// Axis-0 quantization fused with the block means of the FP16 path's block
// selection (ThriftAttention page, Metodologia / 1): one workgroup per
// (head, selection block) unit.  The unit's rows are quantized kMeansRows at a
// time exactly as quantize_axis0_kernel does (whole rows per lane group, so
// the Hadamard butterflies find their partners), and the raw input rows are
// kept in LDS, where one thread per channel adds them in binary64 over
// ascending tokens and divides by the token count: the order and arithmetic
// of block_means_kernel, so the selection is unchanged, without a second pass
// over Q and K.
constexpr int kMeansRows = 128;

template <typename T, bool HAD, bool BAL>
__global__ void __launch_bounds__(256) quantize_means_kernel(QuantArgs A) {
  __shared__ float2_t tab[128];
  __shared__ __align__(16) T raw_rows[kMeansRows * 128];  // [row][channel], cols <= 128
  if (threadIdx.x < 128) tab[threadIdx.x] = kScaleTab.v[threadIdx.x];
  const int64_t bpr = A.cols / 16;
  const int64_t u = blockIdx.x, head = u / A.mnb, ib = u - head * A.mnb;
  const int64_t t0 = ib * A.mblk;
  const int64_t n = (t0 + A.mblk < A.mS ? t0 + A.mblk : A.mS) - t0;
  const int64_t row0 = head * A.mS + t0;
  // the unit's rows lie in one head: the first at row_off(row0), then a fixed step
  const T* x = reinterpret_cast<const T*>(A.x) + A.row_off(row0);
  const int64_t step = A.row_step();
  const int c = threadIdx.x;
  double sum = 0.0;
  constexpr int kMaxPer = kMeansRows * 8 / 256;  // blocks per thread and chunk at cols = 128
  for (int64_t r0 = 0; r0 < n; r0 += kMeansRows) {
    const int64_t nr = n - r0 < kMeansRows ? n - r0 : kMeansRows;
    const int64_t nblk = nr * bpr;
    RawBlock<T> raw[kMaxPer];
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int64_t i = threadIdx.x + 256 * j;
      if (i < nblk) load_raw<T>(raw[j], x + (r0 + i / bpr) * step + (i % bpr) * 16);
    }
    __syncthreads();  // the previous chunk's sums have read the rows; the table is in place
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int64_t i = threadIdx.x + 256 * j;
      if (i < nblk) {
        uint4_t* dst = reinterpret_cast<uint4_t*>(raw_rows + (i / bpr) * A.cols + (i % bpr) * 16);
#pragma unroll
        for (int w = 0; w < RawBlock<T>::N; ++w) dst[w] = raw[j].w[w];
      }
    }
    __syncthreads();
    // the channel sums first: their waves' dependent binary64 adds overlap the
    // other waves' quantization
    if (c < A.cols) {
      int64_t t = 0;
      for (; t + 8 <= nr; t += 8) {
        double v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (double)load_elem<T>(raw_rows + (t + e) * A.cols + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum = sum + v[e];
      }
      for (; t < nr; ++t) sum = sum + (double)load_elem<T>(raw_rows + t * A.cols + c);
    }
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int64_t i = threadIdx.x + 256 * j;
      if (i < nblk) {
        const int64_t rl = i / bpr, cb = i % bpr;
        float y[16];
        raw_to_f32<T>(raw[j], y);
        const int64_t r = row0 + r0 + rl, blk = r * bpr + cb;
        if (BAL) balance_block(y, A, r, cb);
        if (HAD) hadamard_block(y, A, cb, (int)bpr);
        uint32_t codes[2], scale;
        int off;
        quantize_block(y, A.search, A.fmin, A.fmax, tab, codes, scale, off);
        A.codes[blk] = uint2_t{codes[0], codes[1]};
        A.scales[blk] = (uint8_t)scale;
        if (A.offsets) A.offsets[blk] = (int8_t)off;
      }
    }
  }
  if (c < A.cols) A.means[u * A.cols + c] = sum / (double)n;
}

// block_axis 1: one lane per VEC consecutive columns of a group of 16 rows
// (VEC blocks, searched one after the other); consecutive lanes take
// consecutive column groups, so each row load of a wavefront is one
// contiguous segment, and a lane's VEC code bytes of a row pair, its VEC
// scales and its VEC offsets go out as one store each.  VEC is 4 when cols
// and the row step are multiples of 4, else 1.
template <typename T, int VEC>
__device__ __forceinline__ void load_cols(const T* p, float (&v)[VEC]);
template <>
__device__ __forceinline__ void load_cols<uint16_t, 1>(const uint16_t* p, float (&v)[1]) { v[0] = bf16_to_f32(*p); }
template <>
__device__ __forceinline__ void load_cols<half_t, 1>(const half_t* p, float (&v)[1]) { v[0] = (float)*p; }
template <>
__device__ __forceinline__ void load_cols<float, 1>(const float* p, float (&v)[1]) { v[0] = *p; }
template <>
__device__ __forceinline__ void load_cols<uint16_t, 4>(const uint16_t* p, float (&v)[4]) {
  const uint2_t w = *reinterpret_cast<const uint2_t*>(p);
  v[0] = __uint_as_float(w[0] << 16);
  v[1] = __uint_as_float(w[0] & 0xFFFF0000u);
  v[2] = __uint_as_float(w[1] << 16);
  v[3] = __uint_as_float(w[1] & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void load_cols<half_t, 4>(const half_t* p, float (&v)[4]) {
  const half4_t w = *reinterpret_cast<const half4_t*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = (float)w[j];
}
template <>
__device__ __forceinline__ void load_cols<float, 4>(const float* p, float (&v)[4]) {
  const float4_t w = *reinterpret_cast<const float4_t*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = w[j];
}

// VEC bytes (byte j from value j) as one store
template <int VEC>
__device__ __forceinline__ void store_bytes(uint8_t* p, const uint32_t (&b)[VEC]) {
  if constexpr (VEC == 1) {
    *p = (uint8_t)b[0];
  } else {
    *reinterpret_cast<uint32_t*>(p) = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
  }
}

template <typename T, int VEC>
__device__ __forceinline__ void axis1_body(const QuantArgs& A, const float2_t* tab, float ginv, int64_t wg,
                                           int64_t nwg) {
  const int64_t cv = A.cols / VEC;  // column groups per row
  const int64_t nu = (A.rows / 16) * cv;
  const T* x = reinterpret_cast<const T*>(A.x);
  for (int64_t u = wg * blockDim.x + threadIdx.x; u < nu; u += nwg * blockDim.x) {
    const int64_t rb = u / cv, c = (u - rb * cv) * VEC;
    // the blocks' 16 rows lie in one head (heads hold whole blocks)
    const T* xb = x + A.row_off(rb * 16) + c;
    const int64_t step = A.row_step();
    float y[VEC][16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float v[VEC];
      load_cols<T, VEC>(xb + k * step, v);
#pragma unroll
      for (int j = 0; j < VEC; ++j) y[j][k] = A.gmode != 0 ? v[j] * ginv : v[j];
    }
    uint32_t codes[VEC][2], scale[VEC], offb[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      int off;
      quantize_block(y[j], A.search, A.fmin, A.fmax, tab, codes[j], scale[j], off);
      offb[j] = (uint32_t)(off & 0xFF);
    }
    // row pair (2i, 2i+1) of column c + j -> byte i of that block's 8 bytes, at codes8[(rb*8+i)*cols + c + j]
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t b[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) b[j] = (codes[j][i >> 2] >> (8 * (i & 3))) & 0xFFu;
      store_bytes<VEC>(A.codes8 + (rb * 8 + i) * A.cols + c, b);
    }
    const int64_t blk = rb * A.cols + c;
    store_bytes<VEC>(A.scales + blk, scale);
    if (A.offsets) store_bytes<VEC>(reinterpret_cast<uint8_t*>(A.offsets) + blk, offb);
  }
}

template <typename T, int VEC>
__global__ void __launch_bounds__(256) quantize_axis1_kernel(QuantArgs A) {
  __shared__ float2_t tab[128];
  __shared__ float sh[8];
  if (threadIdx.x < 128) tab[threadIdx.x] = kScaleTab.v[threadIdx.x];
  const float ginv = global_factor(A, sh);
  __syncthreads();
  axis1_body<T, VEC>(A, tab, ginv, blockIdx.x, gridDim.x);
}

// Q and K (blocks along d) and V (blocks along rows) of an attention call in
// one launch, when none needs the per-tensor scale, the rotation, the balance
// exponents or the block means: workgroups [0, gq) take Q, [gq, gq + gk) K,
// the rest V, each range striding over its tensor's blocks as its own launch
// would.
struct QkvArgs {
  QuantArgs q, k, v;
  int64_t gq, gk;
  int v4;
};

template <typename T>
__global__ void __launch_bounds__(256) quantize_qkv_kernel(QkvArgs A) {
  __shared__ float2_t tab[128];
  if (threadIdx.x < 128) tab[threadIdx.x] = kScaleTab.v[threadIdx.x];
  __syncthreads();
  const int64_t b = blockIdx.x;
  if (b < A.gq) {
    axis0_body<T, false, false>(A.q, tab, 1.0f, b, A.gq);
  } else if (b < A.gq + A.gk) {
    axis0_body<T, false, false>(A.k, tab, 1.0f, b - A.gq, A.gk);
  } else {
    const int64_t gv = (int64_t)gridDim.x - A.gq - A.gk;
    if (A.v4) axis1_body<T, 4>(A.v, tab, 1.0f, b - A.gq - A.gk, gv);
    else axis1_body<T, 1>(A.v, tab, 1.0f, b - A.gq - A.gk, gv);
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

template <bool HAD, bool BAL>
void launch_axis0(int dtype, int64_t grid, const QuantArgs& A, hipStream_t stream) {
  if (dtype == 0) hipLaunchKernelGGL((quantize_axis0_kernel<uint16_t, HAD, BAL>), dim3(grid), dim3(256), 0, stream, A);
  else if (dtype == 1) hipLaunchKernelGGL((quantize_axis0_kernel<half_t, HAD, BAL>), dim3(grid), dim3(256), 0, stream, A);
  else hipLaunchKernelGGL((quantize_axis0_kernel<float, HAD, BAL>), dim3(grid), dim3(256), 0, stream, A);
}

// ---- magnitude balance exponents -----------------------------------------
// Per (batch, kv head): the rows of Q of its group (G*Sq rows, contiguous) and
// the rows of K (Sk rows, contiguous) are cut into chunks of kBalRows rows;
// a workgroup forms one chunk's binary64 sums of squares per channel (one
// thread per 8 channels and a subset of the rows, then the row groups added in
// order); the finalize kernel adds the chunks in order, divides by the counts
// and decides the exponents.
constexpr int kBalRows = 256;

template <typename T>
__global__ void __launch_bounds__(256) balance_partial_kernel(const T* q, const T* k, TokMap qmap, TokMap kmap,
                                                              int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int d,
                                                              int nchunk, double* partial) {
  __shared__ double red[32][128];
  const int64_t G = H / Hkv;
  const int64_t gi = blockIdx.x;  // ((bk * 2 + side) * nchunk + chunk)
  const int chunk = (int)(gi % nchunk);
  const int side = (int)((gi / nchunk) % 2);
  const int64_t bk = gi / (2 * nchunk);
  const int64_t b = bk / Hkv, hk = bk - b * Hkv;
  const int64_t nrows = side == 0 ? G * Sq : Sk;
  // row r of the side: query head b H + hk G + r / Sq, token r % Sq (Q), or token r of kv head bk (K)
  auto row_ptr = [&](int64_t r) {
    if (side == 0) {
      const int64_t g = r / Sq;
      return q + qmap.head_off(b * H + hk * G + g) + (r - g * Sq) * qmap.ts;
    }
    return k + kmap.head_off(bk) + r * kmap.ts;
  };
  const int per = d / 8;                 // threads per row
  const int rgroups = 256 / per;         // rows in flight per pass (16 or 32)
  const int c0 = (threadIdx.x % per) * 8, rg = threadIdx.x / per;
  double s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.0;
  const int64_t r0 = (int64_t)chunk * kBalRows;
  const int64_t r1 = r0 + kBalRows < nrows ? r0 + kBalRows : nrows;
  for (int64_t r = r0 + rg; r < r1; r += rgroups) {
    const uint4_t w = *reinterpret_cast<const uint4_t*>(row_ptr(r) + c0);
    float y[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (sizeof(T) == 2 && __is_same(T, uint16_t)) {
        y[2 * e] = __uint_as_float(w[e] << 16);
        y[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      } else {
        const half2_t h = __builtin_bit_cast(half2_t, w[e]);
        y[2 * e] = (float)h[0];
        y[2 * e + 1] = (float)h[1];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = s[e] + (double)y[e] * (double)y[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][c0 + e] = s[e];
  __syncthreads();
  if (threadIdx.x < d) {
    double t = 0.0;
    for (int g = 0; g < rgroups; ++g) t = t + red[g][threadIdx.x];
    partial[gi * d + threadIdx.x] = t;
  }
}

// one thread per (batch, kv head, channel)
__global__ void __launch_bounds__(128) balance_exp_kernel(const double* partial, int64_t n_bk, int64_t G,
                                                          int64_t Sq, int64_t Sk, int d, int nchunk,
                                                          int32_t* exps) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_bk * d) return;
  const int64_t bk = i / d;
  const int c = (int)(i - bk * d);
  double sq = 0.0, sk = 0.0;
  const int nq = (int)((G * Sq + kBalRows - 1) / kBalRows), nk = (int)((Sk + kBalRows - 1) / kBalRows);
  for (int ch = 0; ch < nq; ++ch) sq = sq + partial[((bk * 2 + 0) * nchunk + ch) * d + c];
  for (int ch = 0; ch < nk; ++ch) sk = sk + partial[((bk * 2 + 1) * nchunk + ch) * d + c];
  const double mq = sq / (double)(G * Sq), mk = sk / (double)Sk;
  int e = 0;
  if (mq > 0.0 && mk > 0.0) {
    const double A = mq / mk;
    e = 8;
    for (int x = -8; x <= 8; ++x)
      if (__builtin_ldexp(1.0, 2 * (2 * x + 1)) >= A) {
        e = x;
        break;
      }
  }
  exps[i] = e;
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
  if (L.strided && L.gmode == 1) return hipErrorInvalidValue;  // the amax pass reads dense rows
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
  A.cexp = L.cexp;
  A.exp_negate = L.exp_negate;
  A.exp_rows = L.exp_rows > 0 ? L.exp_rows : 1;
  A.means = L.means;
  A.mS = L.mS;
  A.mblk = L.mblk;
  A.mnb = L.mnb;
  A.strided = L.strided;
  A.map = L.map;
  if (L.means) {  // axis 0, bf16/fp16, cols <= 128, no per-tensor scale (checked by the caller)
    const bool had = L.hadamard != 0, bal = L.cexp != nullptr;
    const dim3 g((unsigned)((L.rows / L.mS) * L.mnb));
    if (L.dtype == 0) {
      if (had && bal) hipLaunchKernelGGL((quantize_means_kernel<uint16_t, true, true>), g, dim3(256), 0, stream, A);
      else if (had) hipLaunchKernelGGL((quantize_means_kernel<uint16_t, true, false>), g, dim3(256), 0, stream, A);
      else if (bal) hipLaunchKernelGGL((quantize_means_kernel<uint16_t, false, true>), g, dim3(256), 0, stream, A);
      else hipLaunchKernelGGL((quantize_means_kernel<uint16_t, false, false>), g, dim3(256), 0, stream, A);
    } else {
      if (had && bal) hipLaunchKernelGGL((quantize_means_kernel<half_t, true, true>), g, dim3(256), 0, stream, A);
      else if (had) hipLaunchKernelGGL((quantize_means_kernel<half_t, true, false>), g, dim3(256), 0, stream, A);
      else if (bal) hipLaunchKernelGGL((quantize_means_kernel<half_t, false, true>), g, dim3(256), 0, stream, A);
      else hipLaunchKernelGGL((quantize_means_kernel<half_t, false, false>), g, dim3(256), 0, stream, A);
    }
    return hipGetLastError();
  }
  if (L.axis == 0) {
    const bool had = L.hadamard != 0, bal = L.cexp != nullptr;
    if (had && bal) launch_axis0<true, true>(L.dtype, grid, A, stream);
    else if (had) launch_axis0<true, false>(L.dtype, grid, A, stream);
    else if (bal) launch_axis0<false, true>(L.dtype, grid, A, stream);
    else launch_axis0<false, false>(L.dtype, grid, A, stream);
  } else {
    // four columns per lane when whole groups of 4 stay aligned (codes, scales and offsets rows
    // are cols bytes apart; input rows ld or the map's token stride elements apart)
    const bool v4 = L.cols % 4 == 0 && (L.strided ? L.map.ts % 4 == 0 : L.ld % 4 == 0) &&
                    (reinterpret_cast<uintptr_t>(L.offsets) & 3u) == 0;
    if (v4) {
      const int64_t g4 = ((L.rows / 16) * (L.cols / 4) + 255) / 256;
      const dim3 g((unsigned)(g4 > 2048 ? 2048 : (g4 < 1 ? 1 : g4)));
      if (L.dtype == 0) hipLaunchKernelGGL((quantize_axis1_kernel<uint16_t, 4>), g, dim3(256), 0, stream, A);
      else if (L.dtype == 1) hipLaunchKernelGGL((quantize_axis1_kernel<half_t, 4>), g, dim3(256), 0, stream, A);
      else hipLaunchKernelGGL((quantize_axis1_kernel<float, 4>), g, dim3(256), 0, stream, A);
    } else {
      if (L.dtype == 0) hipLaunchKernelGGL((quantize_axis1_kernel<uint16_t, 1>), dim3(grid), dim3(256), 0, stream, A);
      else if (L.dtype == 1) hipLaunchKernelGGL((quantize_axis1_kernel<half_t, 1>), dim3(grid), dim3(256), 0, stream, A);
      else hipLaunchKernelGGL((quantize_axis1_kernel<float, 1>), dim3(grid), dim3(256), 0, stream, A);
    }
  }
  return hipGetLastError();
}

namespace {
QuantArgs plain_args(const QuantLaunch& L) {
  QuantArgs A;
  A.x = L.x;
  A.rows = L.rows;
  A.cols = L.cols;
  A.ld = L.ld;
  A.codes = reinterpret_cast<uint2_t*>(L.codes);
  A.codes8 = L.codes;
  A.scales = L.scales;
  A.offsets = L.offsets;
  A.g = nullptr;
  A.search = L.search;
  A.fmin = L.fmin;
  A.fmax = L.fmax;
  A.gmode = 0;
  A.amax_part = nullptr;
  A.n_part = 0;
  for (int i = 0; i < 4; ++i) A.hsigns[i] = 0;
  A.hscale = 1.0f;
  A.cexp = nullptr;
  A.exp_negate = 0;
  A.exp_rows = 1;
  A.means = nullptr;
  A.mS = 0;
  A.mblk = 0;
  A.mnb = 0;
  A.strided = L.strided;
  A.map = L.map;
  return A;
}

int64_t part_grid(int64_t work) {
  const int64_t g = (work + 255) / 256;
  return g > 2048 ? 2048 : g;
}
}  // namespace

hipError_t fp4i_launch_quantize_qkv(const QuantLaunch& q, const QuantLaunch& k, const QuantLaunch& v,
                                    hipStream_t stream) {
  for (const QuantLaunch* L : {&q, &k, &v})
    if (L->gmode != 0 || L->g || L->hadamard || L->cexp || L->means || L->dtype != q.dtype || L->dtype == 2)
      return hipErrorInvalidValue;
  if (q.axis != 0 || k.axis != 0 || v.axis != 1) return hipErrorInvalidValue;
  QkvArgs A;
  A.q = plain_args(q);
  A.k = plain_args(k);
  A.v = plain_args(v);
  A.v4 = v.cols % 4 == 0 && (v.strided ? v.map.ts % 4 == 0 : v.ld % 4 == 0) &&
         (reinterpret_cast<uintptr_t>(v.offsets) & 3u) == 0;
  A.gq = part_grid(q.rows * (q.cols / 16));
  A.gk = part_grid(k.rows * (k.cols / 16));
  const int64_t gv = part_grid((v.rows / 16) * (A.v4 ? v.cols / 4 : v.cols));
  const int64_t grid = A.gq + A.gk + gv;
  if (grid == 0) return hipSuccess;
  if (q.dtype == 0) hipLaunchKernelGGL(quantize_qkv_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, stream, A);
  else hipLaunchKernelGGL(quantize_qkv_kernel<half_t>, dim3((unsigned)grid), dim3(256), 0, stream, A);
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

size_t fp4i_balance_partials(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t d) {
  const int64_t G = H / Hkv;
  const int64_t nq = (G * Sq + kBalRows - 1) / kBalRows, nk = (Sk + kBalRows - 1) / kBalRows;
  const int64_t nchunk = nq > nk ? nq : nk;
  return (size_t)(B * Hkv * 2 * nchunk * d);
}

hipError_t fp4i_launch_balance(const BalanceLaunch& L, hipStream_t stream) {
  const int64_t G = L.H / L.Hkv;
  const int64_t nq = (G * L.Sq + kBalRows - 1) / kBalRows, nk = (L.Sk + kBalRows - 1) / kBalRows;
  const int nchunk = (int)(nq > nk ? nq : nk);
  const int64_t n_bk = L.B * L.Hkv;
  const dim3 grid((unsigned)(n_bk * 2 * nchunk));
  if (L.dtype == 0)
    hipLaunchKernelGGL(balance_partial_kernel<uint16_t>, grid, dim3(256), 0, stream, (const uint16_t*)L.q,
                       (const uint16_t*)L.k, L.qmap, L.kmap, L.H, L.Hkv, L.Sq, L.Sk, (int)L.d, nchunk, L.partial);
  else
    hipLaunchKernelGGL(balance_partial_kernel<half_t>, grid, dim3(256), 0, stream, (const half_t*)L.q,
                       (const half_t*)L.k, L.qmap, L.kmap, L.H, L.Hkv, L.Sq, L.Sk, (int)L.d, nchunk, L.partial);
  hipLaunchKernelGGL(balance_exp_kernel, dim3((unsigned)((n_bk * L.d + 127) / 128)), dim3(128), 0, stream, L.partial,
                     n_bk, G, L.Sq, L.Sk, (int)L.d, nchunk, L.exps);
  return hipGetLastError();
}

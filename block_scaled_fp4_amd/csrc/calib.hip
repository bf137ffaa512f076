// calib.hip -- measurement helpers: the achievable rates of the two resources
// the hot path's kernels are priced against (fp16 matrix instructions, HBM
// reads), so that roofline fractions can be stated against measured peaks as
// well as the published ones.  Not part of the computation.
#include <hip/hip_runtime.h>

#include "../../include/fp4_calib.h"
#include "device_common.h"

namespace fp4calib {

using fp4dev::float16_t;
using fp4dev::half_t;
using fp4dev::half8_t;
using fp4dev::uint4_t;

// Every wave runs `iters` rounds of four independent 32x32x16 fp16 MFMA chains
// (no dependency stalls); one float per thread is stored so nothing is dropped.
__global__ void __launch_bounds__(256) mfma_f16_kernel(int64_t iters, float* sink) {
  const half_t x = (half_t)(1.0f + 1e-3f * (threadIdx.x & 7));
  const half8_t a = half8_t{x, x, x, x, x, x, x, x};
  const half8_t b = half8_t{x, -x, x, -x, x, -x, x, -x};
  float16_t acc[4] = {float16_t{0}, float16_t{0}, float16_t{0}, float16_t{0}};
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Streams `n16` 16-byte units once and stores one word per thread.  A wave's
// load covers 1 KiB of contiguous memory; each thread keeps eight loads in
// flight (grid-stride over groups of eight wave-wide rows).
__global__ void __launch_bounds__(256) read_kernel(const uint4_t* __restrict__ src, int64_t n16, uint32_t* sink) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  int64_t i = tid;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const uint4_t v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[tid] = acc;
}

}  // namespace fp4calib

extern "C" {

int fp4_calib_mfma_f16(int64_t iters, int32_t workgroups, float* sink, void* stream) {
  if (iters < 1 || workgroups < 1 || !sink) return -1;
  hipLaunchKernelGGL(fp4calib::mfma_f16_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream, iters,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int fp4_calib_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream) {
  if (!buf || bytes < 16 || bytes % 16 || workgroups < 1 || !sink || (reinterpret_cast<uintptr_t>(buf) & 15u))
    return -1;
  hipLaunchKernelGGL(fp4calib::read_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<const fp4dev::uint4_t*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"

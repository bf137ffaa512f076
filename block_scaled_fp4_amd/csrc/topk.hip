// topk.hip -- block selection for the FP16 path (ThriftAttention page,
// Metodologia / 1): Q and K are cut into blocks of sel_block tokens, every
// block is summarized by its mean token vector, a query/key block pair is
// scored by the dot product of the two means, and each query block keeps its
// top-k visible key blocks.
//
// Means and scores are binary64 with a fixed summation order (ascending tokens,
// ascending channels) so the selection is bit-identical run to run.  The means
// pass streams Q and K once (HBM-bound); the scoring pass is tiny.
#include "device_common.h"
#include "fp4_internal.h"

namespace fp4dev {

template <typename T>
__device__ __forceinline__ double ld_elem(const T* p);
template <>
__device__ __forceinline__ double ld_elem<uint16_t>(const uint16_t* p) { return (double)bf16_to_f32(*p); }
template <>
__device__ __forceinline__ double ld_elem<half_t>(const half_t* p) { return (double)(float)*p; }

// grid: (heads * nblocks); block: d threads, one channel each.
template <typename T>
__global__ void __launch_bounds__(128) block_means_kernel(const T* x, int64_t S, int d, int blk, int nb,
                                                          double* means) {
  const int64_t hb = blockIdx.x;
  const int64_t head = hb / nb, ib = hb - head * nb;
  const int c = threadIdx.x;
  if (c >= d) return;
  const int64_t t0 = ib * blk;
  int64_t t1 = t0 + blk;
  if (t1 > S) t1 = S;
  const T* p = x + (head * S + t0) * d + c;
  double s = 0.0;
  int64_t n = t1 - t0;
  int64_t t = 0;
  for (; t + 8 <= n; t += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ld_elem<T>(p + (t + u) * d);
#pragma unroll
    for (int u = 0; u < 8; ++u) s = s + v[u];
  }
  for (; t < n; ++t) s = s + ld_elem<T>(p + t * d);
  means[hb * d + c] = s / (double)n;
}

// grid: (B*H*nqb); block: 256 threads.  Scores every visible key block, ranks
// them (descending score, ascending index on ties) and writes the kept ones in
// ascending order, padded with -1.
__global__ void __launch_bounds__(256) block_topk_kernel(const double* qm, const double* km, int64_t H,
                                                         int64_t Hkv, int nqb, int nkb, int d, int causal,
                                                         int pct, int kmax, int32_t* idx, int32_t* cnt) {
  extern __shared__ double smem[];  // [d] query mean, [nkb] scores, [nkb] kept flags
  double* qv = smem;
  double* sc = smem + d;
  int* kept = reinterpret_cast<int*>(smem + d + nkb);
  const int64_t g = blockIdx.x;  // (b*H + h) * nqb + i
  const int64_t bh = g / nqb;
  const int i = (int)(g - bh * nqb);
  const int64_t b = bh / H, h = bh - b * H;
  const int64_t hk = h / (H / Hkv);
  const double* kmh = km + (b * Hkv + hk) * (int64_t)nkb * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) qv[c] = qm[g * d + c];
  __syncthreads();
  const int nvis = causal ? (i + 1 < nkb ? i + 1 : nkb) : nkb;
  const int k = (pct * nvis + 99) / 100;
  for (int j = threadIdx.x; j < nvis; j += blockDim.x) {
    double s = 0.0;
    const double* kv = kmh + (int64_t)j * d;
    for (int c = 0; c < d; ++c) {
      double p = __dmul_rn(qv[c], kv[c]);
      s = __dadd_rn(s, p);
    }
    sc[j] = s;
  }
  __syncthreads();
  int32_t* out = idx + g * kmax;
  // rank of j = number of visible j' ahead of it; kept iff rank < k
  for (int j = threadIdx.x; j < nvis; j += blockDim.x) {
    const double sj = sc[j];
    int rank = 0;
    for (int jj = 0; jj < nvis; ++jj) {
      const double so = sc[jj];
      rank += (so > sj || (so == sj && jj < j)) ? 1 : 0;
    }
    kept[j] = rank < k ? 1 : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int w = 0;
    for (int j = 0; j < nvis; ++j)
      if (kept[j]) out[w++] = j;
    for (int t = w; t < kmax; ++t) out[t] = -1;
    cnt[g] = k;
  }
}

}  // namespace fp4dev

using namespace fp4dev;

hipError_t fp4i_launch_topk(const TopkLaunch& L, hipStream_t stream) {
  const int d = (int)L.d;
  const int64_t gq = L.B * L.H * L.nqb, gk = L.B * L.Hkv * L.nkb;
  if (L.dtype == 0) {
    hipLaunchKernelGGL(block_means_kernel<uint16_t>, dim3(gq), dim3(d), 0, stream, (const uint16_t*)L.q, L.Sq, d,
                       L.sel_block, L.nqb, L.qmeans);
    hipLaunchKernelGGL(block_means_kernel<uint16_t>, dim3(gk), dim3(d), 0, stream, (const uint16_t*)L.k, L.Sk, d,
                       L.sel_block, L.nkb, L.kmeans);
  } else {
    hipLaunchKernelGGL(block_means_kernel<half_t>, dim3(gq), dim3(d), 0, stream, (const half_t*)L.q, L.Sq, d,
                       L.sel_block, L.nqb, L.qmeans);
    hipLaunchKernelGGL(block_means_kernel<half_t>, dim3(gk), dim3(d), 0, stream, (const half_t*)L.k, L.Sk, d,
                       L.sel_block, L.nkb, L.kmeans);
  }
  size_t shm = sizeof(double) * (size_t)(d + L.nkb) + sizeof(int) * (size_t)L.nkb;
  hipLaunchKernelGGL(block_topk_kernel, dim3(gq), dim3(256), shm, stream, L.qmeans, L.kmeans, L.H, L.Hkv, L.nqb,
                     L.nkb, d, L.causal, L.pct, L.kmax, L.idx, L.cnt);
  return hipGetLastError();
}

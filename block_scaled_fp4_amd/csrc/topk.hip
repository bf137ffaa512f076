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

// ---- decode: promoted middle blocks of one query token per query head ----
//
// The query block of a kv head is its G query vectors; its mean and the
// key-block means (cached binary64 sums over each block's tokens, divided by
// their count) give one binary64 score per middle block, summed over
// ascending channels.  The ceil(pct * n / 100) best blocks (descending score,
// lower block first on ties) are kept.
//   decode_scores_kernel: 32 blocks per workgroup; the sums are read
//     coalesced (a wavefront reads 512 contiguous bytes), each channel's
//     product goes to LDS, then one lane per block adds its row in order;
//   decode_select_kernel: one workgroup per (batch, kv head): a radix select
//     (8 passes of 8 bits) on order-preserving 64-bit keys of the scores, kept
//     in LDS when they fit, then the kept blocks in ascending order and a bit
//     mask of the same set.

constexpr int kScoreBlocks = 32;    // middle blocks per scoring workgroup
constexpr int kSelLdsKeys = 4096;   // keys the select kernel keeps in LDS

// Scores as unsigned keys that order like the doubles (-0 folded into +0).
__device__ __forceinline__ uint64_t score_key(double s) {
  if (s == 0.0) s = 0.0;
  const uint64_t u = (uint64_t)__double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

struct DecSelArgs {
  const uint16_t* q;
  const double* k_sum;
  const int32_t* mid_len;
  int64_t Hkv, mid_cap;
  int G, d, pct, kmax, nbc, nbw;
  uint64_t* keys;
  int32_t* idx;
  int32_t* cnt;
  uint32_t* mask;
};

__device__ __forceinline__ int64_t sel_mid_len(const DecSelArgs& A, int64_t b) {
  int64_t M = A.mid_cap > 0 ? A.mid_len[b] : 0;  // (no middle region: mid_len may be absent)
  if (M < 0) M = 0;
  if (M > A.mid_cap) M = A.mid_cap;
  return M & ~(int64_t)15;
}

// grid: B*Hkv*ceil(nbc/32); block: 256 threads.
__global__ void __launch_bounds__(256) decode_scores_kernel(DecSelArgs A) {
  __shared__ double qm[128];
  __shared__ double prod[kScoreBlocks][129];  // one pad column: lanes summing rows hit distinct banks
  const int tid = threadIdx.x;
  const int nchunk = (A.nbc + kScoreBlocks - 1) / kScoreBlocks;
  const int64_t bk = blockIdx.x / nchunk;
  const int j0 = (int)(blockIdx.x % nchunk) * kScoreBlocks;
  const int64_t M = sel_mid_len(A, bk / A.Hkv);
  const int nb = (int)((M + kDecSelBlock - 1) / kDecSelBlock);
  if (j0 >= nb) return;
  const int d = A.d;
  const int nloc = nb - j0 < kScoreBlocks ? nb - j0 : kScoreBlocks;
  const double* base = A.k_sum + (bk * A.nbc + j0) * d;
  // the sums first (in flight while the query mean is formed): element pairs
  // e = 2*tid + 512*i of the workgroup's rows
  constexpr int kPer = kScoreBlocks * 128 / 512;
  double2_t w[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = 2 * tid + 512 * i;
    w[i] = e < nloc * d ? *reinterpret_cast<const double2_t*>(base + e) : double2_t{0.0, 0.0};
  }
  for (int c = tid; c < d; c += 256) {
    double s = 0.0;
    for (int g = 0; g < A.G; ++g) s = __dadd_rn(s, (double)bf16_to_f32(A.q[(bk * A.G + g) * d + c]));
    qm[c] = __ddiv_rn(s, (double)A.G);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = 2 * tid + 512 * i;
    if (e >= nloc * d) break;
    const int jb = e / d, c = e % d;  // c even: the pair (c, c+1) stays in one row
    const int64_t t0 = (int64_t)(j0 + jb) * kDecSelBlock;
    const int n = (int)(M - t0 < kDecSelBlock ? M - t0 : kDecSelBlock);
    double m0, m1;
    if ((n & (n - 1)) == 0) {  // a power of two: sum * (1/n) is the exact quotient
      const double rn = 1.0 / (double)n;
      m0 = __dmul_rn(w[i][0], rn);
      m1 = __dmul_rn(w[i][1], rn);
    } else {
      m0 = __ddiv_rn(w[i][0], (double)n);
      m1 = __ddiv_rn(w[i][1], (double)n);
    }
    prod[jb][c] = __dmul_rn(qm[c], m0);
    prod[jb][c + 1] = __dmul_rn(qm[c + 1], m1);
  }
  __syncthreads();
  if (tid < nloc) {
    // 16 row entries are read ahead of each run of additions (the adds stay
    // in channel order)
    double s = 0.0;
    for (int c0 = 0; c0 < d; c0 += 16) {
      double r[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) r[i] = prod[tid][c0 + i];
#pragma unroll
      for (int i = 0; i < 16; ++i) s = __dadd_rn(s, r[i]);
    }
    A.keys[bk * A.nbc + j0 + tid] = score_key(s);
  }
}

// grid: B*Hkv; block: 256 threads.  KEYS_IN_LDS: nb <= kSelLdsKeys.
template <bool KEYS_IN_LDS>
__global__ void __launch_bounds__(256) decode_select_kernel(DecSelArgs A) {
  __shared__ uint64_t lkeys[KEYS_IN_LDS ? kSelLdsKeys : 1];
  __shared__ int hist[256];
  __shared__ int wtot[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bk = blockIdx.x;
  const int64_t M = sel_mid_len(A, bk / A.Hkv);
  const int nb = (int)((M + kDecSelBlock - 1) / kDecSelBlock);
  const int k = (A.pct * nb + 99) / 100;
  const uint64_t* gkeys = A.keys + bk * A.nbc;
  if (KEYS_IN_LDS)
    for (int j = tid; j < nb; j += 256) lkeys[j] = gkeys[j];
  __syncthreads();
  auto key = [&](int j) { return KEYS_IN_LDS ? lkeys[j] : gkeys[j]; };
  // k-th largest key: after the passes `prefix` is its value and `rem` the
  // number of keys equal to it that are kept (the lowest blocks among them)
  uint64_t prefix = 0;
  int rem = k;
  if (k > 0) {
    for (int shift = 56; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      const uint64_t hi = shift == 56 ? 0ull : (~0ull << (shift + 8));
      for (int j = tid; j < nb; j += 256) {
        const uint64_t u = key(j);
        if ((u & hi) == prefix) atomicAdd(&hist[(int)((u >> shift) & 255u)], 1);
      }
      __syncthreads();
      // every wave scans the 256 bins from the top: lane l holds bins 255-4l .. 252-4l
      int c4[4], own = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c4[i] = hist[255 - 4 * lane - i];
        own += c4[i];
      }
      int incl = own;  // inclusive prefix over lanes (descending bins)
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const int excl = incl - own;
      // the lane whose range crosses rem finds the bin
      int found = -1, above = 0;
      if (excl < rem && incl >= rem) {
        int acc = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (found < 0 && acc + c4[i] >= rem) {
            found = 255 - 4 * lane - i;
            above = acc;
          }
          acc += c4[i];
        }
      }
      const unsigned long long who = __ballot(found >= 0);
      const int src = (int)__builtin_ctzll(who);
      const int bin = __shfl(found, src, 64);
      rem -= __shfl(above, src, 64);
      prefix |= (uint64_t)bin << shift;
      __syncthreads();
    }
  }
  // kept blocks in ascending order, with the bit mask
  int32_t* out = A.idx + bk * A.kmax;
  uint32_t* mask = A.mask + bk * A.nbw;
  const uint64_t below = (1ull << lane) - 1ull;
  int run_tie = 0, run_sel = 0;
  for (int base = 0; base < nb; base += 256) {
    const int j = base + tid;
    const uint64_t u = j < nb ? key(j) : 0ull;
    const bool tie = k > 0 && j < nb && u == prefix;
    const unsigned long long bt = __ballot(tie);
    if (lane == 0) wtot[0][wave] = __popcll(bt);
    __syncthreads();
    int off_t = run_tie, all_t = 0;
    for (int w = 0; w < 4; ++w) {
      off_t += w < wave ? wtot[0][w] : 0;
      all_t += wtot[0][w];
    }
    const bool sel = k > 0 && j < nb && (u > prefix || (tie && off_t + __popcll(bt & below) < rem));
    const unsigned long long bs = __ballot(sel);
    if (lane == 0) wtot[1][wave] = __popcll(bs);
    __syncthreads();
    int off_s = run_sel, all_s = 0;
    for (int w = 0; w < 4; ++w) {
      off_s += w < wave ? wtot[1][w] : 0;
      all_s += wtot[1][w];
    }
    if (sel) out[off_s + __popcll(bs & below)] = j;
    if ((lane & 31) == 0 && j < nb) mask[j >> 5] = (uint32_t)(bs >> (lane & 32));
    run_tie += all_t;
    run_sel += all_s;
    __syncthreads();
  }
  for (int p = k + tid; p < A.kmax; p += 256) out[p] = -1;
  if (tid == 0) A.cnt[bk] = k;
}

}  // namespace fp4dev

using namespace fp4dev;

hipError_t fp4i_launch_decode_select(const DecSelectLaunch& L, hipStream_t stream) {
  DecSelArgs A;
  A.q = (const uint16_t*)L.q;
  A.k_sum = L.k_sum;
  A.mid_len = L.mid_len;
  A.Hkv = L.Hkv;
  A.mid_cap = L.mid_cap;
  A.G = (int)(L.Hq / L.Hkv);
  A.d = (int)L.d;
  A.pct = L.pct;
  A.kmax = L.kmax;
  A.nbc = L.nbc;
  A.nbw = L.nbw;
  A.keys = L.keys;
  A.idx = L.idx;
  A.cnt = L.cnt;
  A.mask = L.mask;
  const int64_t nbk = L.B * L.Hkv;
  if (L.nbc > 0) {
    const int nchunk = (L.nbc + kScoreBlocks - 1) / kScoreBlocks;
    hipLaunchKernelGGL(decode_scores_kernel, dim3((unsigned)(nbk * nchunk)), dim3(256), 0, stream, A);
  }
  if (L.nbc <= kSelLdsKeys)
    hipLaunchKernelGGL(decode_select_kernel<true>, dim3((unsigned)nbk), dim3(256), 0, stream, A);
  else
    hipLaunchKernelGGL(decode_select_kernel<false>, dim3((unsigned)nbk), dim3(256), 0, stream, A);
  return hipGetLastError();
}

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

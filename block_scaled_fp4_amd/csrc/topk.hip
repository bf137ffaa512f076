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

// Element e (0..7) of 8 consecutive bf16 / fp16 values in 16 bytes, exactly.
template <typename T>
__device__ __forceinline__ double elem8(const uint4_t& w, int e);
template <>
__device__ __forceinline__ double elem8<uint16_t>(const uint4_t& w, int e) {
  const uint32_t v = w[e >> 1];
  return (double)__uint_as_float((e & 1) ? (v & 0xFFFF0000u) : (v << 16));
}
template <>
__device__ __forceinline__ double elem8<half_t>(const uint4_t& w, int e) {
  const uint32_t v = w[e >> 1];
  return (double)(float)__builtin_bit_cast(half_t, (uint16_t)((e & 1) ? (v >> 16) : (v & 0xFFFFu)));
}

// Block means: one thread per 8 channels of one (head, block), 16-byte loads
// (sixteen in flight), each channel summed over ascending tokens in binary64
// and divided by the token count.  One launch covers the Q units and then the
// K units; 256 threads cover 256 / (d / 8) units.
template <typename T>
struct MeansArgs {
  const T *q, *k;
  TokMap qmap, kmap;  // row offsets of q and k
  int64_t Sq, Sk, nunits_q, nunits_k;
  int d, blk, nqb, nkb;
  double *qmeans, *kmeans;
};

template <typename T>
__global__ void __launch_bounds__(256) block_means_kernel(MeansArgs<T> A) {
  const int per = A.d / 8;
  int64_t u = (int64_t)blockIdx.x * (256 / per) + threadIdx.x / per;
  const bool isq = u < A.nunits_q;
  if (!isq) u -= A.nunits_q;
  if (!isq && u >= A.nunits_k) return;
  const T* x = isq ? A.q : A.k;
  const TokMap& map = isq ? A.qmap : A.kmap;
  const int64_t S = isq ? A.Sq : A.Sk;
  const int nb = isq ? A.nqb : A.nkb;
  double* means = isq ? A.qmeans : A.kmeans;
  const int d = A.d, blk = A.blk;
  const int c0 = (threadIdx.x % per) * 8;
  const int64_t head = u / nb, ib = u - head * nb;
  const int64_t t0 = ib * blk;
  const int64_t n = (t0 + blk < S ? t0 + blk : S) - t0;
  const T* p = x + map.head_off(head) + t0 * map.ts + c0;
  const int64_t ts = map.ts;
  double s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.0;
  int64_t t = 0;
  for (; t + 16 <= n; t += 16) {
    uint4_t w[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) w[v] = *reinterpret_cast<const uint4_t*>(p + (t + v) * ts);
#pragma unroll
    for (int v = 0; v < 16; ++v)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = s[e] + elem8<T>(w[v], e);
  }
  for (; t < n; ++t) {
    const uint4_t w = *reinterpret_cast<const uint4_t*>(p + t * ts);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = s[e] + elem8<T>(w, e);
  }
  double* out = means + u * d + c0;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = s[e] / (double)n;
}

// Scores of 16 query blocks x 64 key blocks of one (batch, head) per
// workgroup.  Wave w takes query blocks i0 + 4w .. +3, whose means are the
// same for all its lanes and are read through the scalar unit; lane l takes
// key block j0 + l, from a transposed LDS image of the 64 key means (32
// channels at a time, staged from coalesced reads).  Every score is one
// binary64 fused multiply-add per channel in ascending channel order, written
// as an order-preserving 64-bit key.  A tile wholly above the causal
// diagonal does nothing; its keys are never read.  The fixed channel order
// makes every score one chain of d dependent fused multiply-adds: a causal 32K
// prefill has about 20 such chains per SIMD in all, where the fp64 unit needs
// about 64 in flight to run at its rate, so the chains' latency sets the time.
constexpr int kScQ = 16, kScK = 64, kScC = 32;

// Scores as unsigned keys that order like the doubles (-0 folded into +0).
__device__ __forceinline__ uint64_t score_key(double s) {
  if (s == 0.0) s = 0.0;
  const uint64_t u = (uint64_t)__double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__global__ void __launch_bounds__(256) block_scores_kernel(const double* __restrict__ qm,
                                                           const double* __restrict__ km, int64_t H, int64_t Hkv,
                                                           int nqb, int nkb, int d, int causal, int ntq, int ntk,
                                                           uint64_t* __restrict__ keys) {
  __shared__ double skt[kScC][kScK + 1];  // [channel][key block]
  // Workgroups go to the 8 XCDs in turn (blockIdx modulo 8): consecutive
  // tiles -- one head's -- are given to one XCD, so the key means its tiles
  // all re-read stay in that XCD's L2.
  const unsigned per = gridDim.x / 8;
  const unsigned lin = blockIdx.x < 8 * per ? (blockIdx.x % 8) * per + blockIdx.x / 8 : blockIdx.x;
  const int64_t bh = lin / (ntq * ntk);
  const int tile = (int)(lin - bh * ntq * ntk);
  const int i0 = (tile / ntk) * kScQ, j0 = (tile % ntk) * kScK;
  const int ilast = i0 + kScQ - 1 < nqb - 1 ? i0 + kScQ - 1 : nqb - 1;
  if (causal && j0 > ilast) return;
  const int64_t b = bh / H, h = bh - b * H, hk = h / (H / Hkv);
  const double* qb = qm + bh * nqb * d;
  const double* kb = km + (b * Hkv + hk) * nkb * d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int iw = i0 + 4 * __builtin_amdgcn_readfirstlane(tid >> 6);  // this wave's first query block
  const int iwl = iw + 3 < nqb - 1 ? iw + 3 : nqb - 1;                // its last one that exists
  const bool live = iw < nqb && (!causal || j0 <= iwl);
  // query blocks past the last one read the last one (their scores are not written)
  const double* qr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) qr[r] = qb + (int64_t)(iw + r < nqb ? iw + r : nqb - 1) * d;
  // staging: element e = tid + 256 u of a chunk -> key block e / 32, channel e % 32
  constexpr int NK = kScK * kScC / 256;
  double rk[NK];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int e = tid + 256 * u, r = e / kScC, cc = e % kScC;
      rk[u] = j0 + r < nkb ? kb[(int64_t)(j0 + r) * d + c0 + cc] : 0.0;
    }
  };
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  fetch(0);
  for (int c0 = 0; c0 < d; c0 += kScC) {
    __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int e = tid + 256 * u;
      skt[e % kScC][e / kScC] = rk[u];
    }
    __syncthreads();
    if (c0 + kScC < d) fetch(c0 + kScC);
    if (live) {
      // eight channels at a time (each score takes them in ascending
      // order); the query means of the next eight are loaded before this
      // group's arithmetic
      double qv[4][8], qn[4][8];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) qv[r][j] = qr[r][c0 + j];
#pragma unroll
      for (int c8 = 0; c8 < kScC; c8 += 8) {
        if (c8 + 8 < kScC) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j) qn[r][j] = qr[r][c0 + c8 + 8 + j];
        }
        double kv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) kv[j] = skt[c8 + j][lane];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] = __fma_rn(qv[r][j], kv[j], acc[r]);
        if (c8 + 8 < kScC) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j) qv[r][j] = qn[r][j];
        }
      }
    }
  }
  const int j = j0 + lane;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = iw + r;
    if (live && i < nqb && j < nkb && (!causal || j <= i)) keys[(bh * nqb + i) * nkb + j] = score_key(acc[r]);
  }
}

// ---- decode: promoted middle blocks of one query token per query head ----
//
// The query block of a kv head is its G query vectors; its mean and the
// key-block means (cached binary64 sums over each block's tokens, divided by
// their count) give one binary64 score per middle block, one fused
// multiply-add per channel in ascending order.  The ceil(pct * n / 100) best
// blocks (descending score, lower block first on ties) are kept.
//   decode_scores_kernel: 16 blocks per workgroup; the sums are read
//     coalesced (a wavefront reads 512 contiguous bytes), each block's mean
//     goes to LDS, then one lane per block runs its row in channel order;
//   decode_select_kernel: one workgroup per (batch, kv head): a radix select
//     (8 passes of 8 bits) on order-preserving 64-bit keys of the scores, kept
//     in LDS when they fit, then the kept blocks in ascending order and a bit
//     mask of the same set.

constexpr int kScoreBlocks = 16;    // middle blocks per scoring workgroup (17 KB of LDS: eight workgroups per CU)
constexpr int kSelLdsKeys = 4096;   // keys the select kernel keeps in LDS


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
  __shared__ double kmr[kScoreBlocks][129];  // block means; one pad column: lanes reading rows hit distinct banks
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
    kmr[jb][c] = m0;
    kmr[jb][c + 1] = m1;
  }
  __syncthreads();
  if (tid < nloc) {
    // one fused multiply-add per channel in ascending order; 16 row entries
    // are read ahead of each run
    double s = 0.0;
    for (int c0 = 0; c0 < d; c0 += 16) {
      double r[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) r[i] = kmr[tid][c0 + i];
#pragma unroll
      for (int i = 0; i < 16; ++i) s = __fma_rn(qm[c0 + i], r[i], s);
    }
    A.keys[bk * A.nbc + j0 + tid] = score_key(s);
  }
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within each
// 16-lane row, then row 0's total into row 1 and row 2's into row 3, then
// the total of rows 0-1 into rows 2-3 (lanes whose source is out of range add
// zero).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// The k largest of keys[0..nb) (ties: the lower index first), by a radix
// select over 8-bit digits, stopping at the first digit whose threshold bin
// is kept whole: the kept indices go to out[0..k) in ascending order and
// out[k..kmax) gets -1; mask (nullable) gets the same set as bits.  Called by
// all 256 threads of the workgroup (block-wide barriers inside).
__device__ void select_top_keys(const uint64_t* keys, int nb, int k, int kmax, int32_t* out, uint32_t* mask) {
  __shared__ int hist[256];
  __shared__ int wtot[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // k-th largest key: after the passes `prefix` is its value and `rem` the
  // number of keys equal to it that are kept (the lowest indices among them)
  uint64_t prefix = 0;
  int rem = k, fshift = 0;  // the threshold is decided on the key bits from fshift up
  if (k > 0) {
    for (int shift = 56; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      const uint64_t hi = shift == 56 ? 0ull : (~0ull << (shift + 8));
      for (int j = tid; j < nb; j += 256) {
        const uint64_t u = keys[j];
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
      const int incl = wave_incl_scan(own);  // inclusive prefix over lanes (descending bins)
      const int excl = incl - own;
      // the lane whose range crosses rem finds the bin
      int found = -1, above = 0, fcnt = 0;
      if (excl < rem && incl >= rem) {
        int acc = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (found < 0 && acc + c4[i] >= rem) {
            found = 255 - 4 * lane - i;
            above = acc;
            fcnt = c4[i];
          }
          acc += c4[i];
        }
      }
      const unsigned long long who = __ballot(found >= 0);
      const int src = (int)__builtin_ctzll(who);
      const int bin = __builtin_amdgcn_readlane(found, src);
      rem -= __builtin_amdgcn_readlane(above, src);
      prefix |= (uint64_t)bin << shift;
      fshift = shift;
      __syncthreads();
      // every key of the threshold's bin is kept: no lower digit can matter
      // (every wave scanned the same histogram, so all leave together)
      if (__builtin_amdgcn_readlane(fcnt, src) == rem) break;
    }
  }
  // kept indices in ascending order (and the bit mask)
  const uint64_t below = (1ull << lane) - 1ull;
  int run_tie = 0, run_sel = 0;
  for (int base = 0; base < nb; base += 256) {
    const int j = base + tid;
    const uint64_t u = j < nb ? keys[j] : 0ull;
    const uint64_t uh = u >> fshift, ph = prefix >> fshift;
    const bool tie = k > 0 && j < nb && uh == ph;
    const unsigned long long bt = __ballot(tie);
    if (lane == 0) wtot[0][wave] = __popcll(bt);
    __syncthreads();
    int off_t = run_tie, all_t = 0;
    for (int w = 0; w < 4; ++w) {
      off_t += w < wave ? wtot[0][w] : 0;
      all_t += wtot[0][w];
    }
    const bool sel = k > 0 && j < nb && (uh > ph || (tie && off_t + __popcll(bt & below) < rem));
    const unsigned long long bs = __ballot(sel);
    if (lane == 0) wtot[1][wave] = __popcll(bs);
    __syncthreads();
    int off_s = run_sel, all_s = 0;
    for (int w = 0; w < 4; ++w) {
      off_s += w < wave ? wtot[1][w] : 0;
      all_s += wtot[1][w];
    }
    if (sel) out[off_s + __popcll(bs & below)] = j;
    if (mask && (lane & 31) == 0 && j < nb) mask[j >> 5] = (uint32_t)(bs >> (lane & 32));
    run_tie += all_t;
    run_sel += all_s;
    __syncthreads();
  }
  for (int p = k + tid; p < kmax; p += 256) out[p] = -1;
}

// grid: B*Hkv; block: 256 threads.  KEYS_IN_LDS: nb <= kSelLdsKeys.
template <bool KEYS_IN_LDS>
__global__ void __launch_bounds__(256) decode_select_kernel(DecSelArgs A) {
  __shared__ uint64_t lkeys[KEYS_IN_LDS ? kSelLdsKeys : 1];
  const int tid = threadIdx.x;
  const int64_t bk = blockIdx.x;
  const int64_t M = sel_mid_len(A, bk / A.Hkv);
  const int nb = (int)((M + kDecSelBlock - 1) / kDecSelBlock);
  const int k = (A.pct * nb + 99) / 100;
  const uint64_t* gkeys = A.keys + bk * A.nbc;
  if (KEYS_IN_LDS)
    for (int j = tid; j < nb; j += 256) lkeys[j] = gkeys[j];
  __syncthreads();
  select_top_keys(KEYS_IN_LDS ? lkeys : gkeys, nb, k, A.kmax, A.idx + bk * A.kmax, A.mask + bk * A.nbw);
  if (tid == 0) A.cnt[bk] = k;
}

// Prefill selection, one wave per (batch, head, query block) row, no
// workgroup barrier: a radix select over 8-bit digits of the row's visible
// keys (from block_scores_kernel) with a per-wave histogram in LDS, stopping
// at the first digit whose threshold bin is kept whole, then the kept indices
// in ascending order (the k largest, ties to the lower index), -1 padding and
// the count.  Rows of at most kSelRegKeys visible blocks are
// read once into registers (four keys per lane); longer rows are read from
// memory in every pass.
constexpr int kSelRegKeys = 256;

// One 64-key chunk of the final emission: keys whose bits from `shift` up
// exceed the threshold's, and ties there while fewer than rem have been
// kept (the lower indices first).
__device__ __forceinline__ void select_emit(uint64_t u, bool in, int j, int k, int nvis, uint64_t prefix, int shift,
                                            int rem, int lane, int& run_tie, int& run_sel, int32_t* out) {
  const uint64_t below = (1ull << lane) - 1ull;
  bool sel;
  if (k >= nvis) {
    sel = in;
  } else {
    const uint64_t uh = u >> shift, ph = prefix >> shift;
    const bool tie = k > 0 && in && uh == ph;
    const unsigned long long bt = __ballot(tie);
    sel = k > 0 && in && (uh > ph || (tie && run_tie + __popcll(bt & below) < rem));
    run_tie += __popcll(bt);
  }
  const unsigned long long bs = __ballot(sel);
  if (sel) out[run_sel + __popcll(bs & below)] = j;
  run_sel += __popcll(bs);
}

__global__ void __launch_bounds__(256) block_select_kernel(const uint64_t* keys, int64_t nrows, int nqb, int nkb,
                                                           int causal, int pct, int kmax, int32_t* idx,
                                                           int32_t* cnt) {
  __shared__ int hist[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t g = (int64_t)blockIdx.x * 4 + wave;  // (b*H + h) * nqb + i
  if (g >= nrows) return;
  const int i = (int)(g % nqb);
  const int nvis = causal ? (i + 1 < nkb ? i + 1 : nkb) : nkb;
  const int k = (pct * nvis + 99) / 100;
  const uint64_t* row = keys + g * nkb;
  const bool inreg = nvis <= kSelRegKeys;
  constexpr int NR = kSelRegKeys / 64;
  uint64_t kv[NR];
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    const int j = lane + 64 * q;
    kv[q] = inreg && j < nvis ? row[j] : 0ull;
  }
  int* hw = hist[wave];
  uint64_t prefix = 0;
  int rem = k, fshift = 0;  // the threshold is decided on the key bits from fshift up
  if (k > 0 && k < nvis) {
    for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) hw[lane + 64 * q] = 0;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const uint64_t hi = shift == 56 ? 0ull : (~0ull << (shift + 8));
      if (inreg) {
#pragma unroll
        for (int q = 0; q < NR; ++q) {
          const uint64_t u = kv[q];
          if (lane + 64 * q < nvis && (u & hi) == prefix) atomicAdd(&hw[(int)((u >> shift) & 255u)], 1);
        }
      } else {
        for (int j = lane; j < nvis; j += 64) {
          const uint64_t u = row[j];
          if ((u & hi) == prefix) atomicAdd(&hw[(int)((u >> shift) & 255u)], 1);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      // lane l holds bins 255-4l .. 252-4l (scanned from the top)
      int c4[4], own = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c4[q] = hw[255 - 4 * lane - q];
        own += c4[q];
      }
      const int incl = wave_incl_scan(own);
      const int excl = incl - own;
      int found = -1, above = 0, fcnt = 0;
      if (excl < rem && incl >= rem) {
        int acc = excl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (found < 0 && acc + c4[q] >= rem) {
            found = 255 - 4 * lane - q;
            above = acc;
            fcnt = c4[q];
          }
          acc += c4[q];
        }
      }
      const unsigned long long who = __ballot(found >= 0);
      const int src = (int)__builtin_ctzll(who);
      prefix |= (uint64_t)__builtin_amdgcn_readlane(found, src) << shift;
      rem -= __builtin_amdgcn_readlane(above, src);
      fshift = shift;
      // the next pass clears this histogram: all reads of it are done first
      __builtin_amdgcn_wave_barrier();
      // every key of the threshold's bin is kept: no lower digit can matter
      if (__builtin_amdgcn_readlane(fcnt, src) == rem) break;
    }
  }
  // kept: every visible block when k >= nvis; else keys above the threshold
  // and the first rem ties
  int32_t* out = idx + g * kmax;
  int run_tie = 0, run_sel = 0;
  if (inreg) {
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int j = 64 * q + lane;
      select_emit(kv[q], j < nvis, j, k, nvis, prefix, fshift, rem, lane, run_tie, run_sel, out);
    }
  } else {
    for (int base = 0; base < nvis; base += 64) {
      const int j = base + lane;
      const bool in = j < nvis;
      select_emit(in ? row[j] : 0ull, in, j, k, nvis, prefix, fshift, rem, lane, run_tie, run_sel, out);
    }
  }
  for (int p = k + lane; p < kmax; p += 64) out[p] = -1;
  if (lane == 0) cnt[g] = k;
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

template <typename T>
hipError_t launch_means(const TopkLaunch& L, hipStream_t stream) {
  MeansArgs<T> A;
  A.q = (const T*)L.q;
  A.k = (const T*)L.k;
  A.Sq = L.Sq;
  A.Sk = L.Sk;
  A.nunits_q = L.B * L.H * L.nqb;
  A.nunits_k = L.B * L.Hkv * L.nkb;
  A.d = (int)L.d;
  A.blk = L.sel_block;
  A.nqb = L.nqb;
  A.nkb = L.nkb;
  A.qmap = L.qmap;
  A.kmap = L.kmap;
  A.qmeans = L.qmeans;
  A.kmeans = L.kmeans;
  const int upw = 256 / (A.d / 8);  // (head, block) units per workgroup
  const int64_t units = A.nunits_q + A.nunits_k;
  hipLaunchKernelGGL(block_means_kernel<T>, dim3((unsigned)((units + upw - 1) / upw)), dim3(256), 0, stream, A);
  return hipGetLastError();
}

hipError_t fp4i_launch_topk(const TopkLaunch& L, hipStream_t stream) {
  const int d = (int)L.d;
  const int64_t gq = L.B * L.H * L.nqb;
  if (!L.means_ready) {
    const hipError_t e = L.dtype == 0 ? launch_means<uint16_t>(L, stream) : launch_means<half_t>(L, stream);
    if (e != hipSuccess) return e;
  }
  const int ntq = (L.nqb + kScQ - 1) / kScQ, ntk = (L.nkb + kScK - 1) / kScK;
  hipLaunchKernelGGL(block_scores_kernel, dim3((unsigned)(L.B * L.H * ntq * ntk)), dim3(256), 0, stream, L.qmeans,
                     L.kmeans, L.H, L.Hkv, L.nqb, L.nkb, d, L.causal, ntq, ntk, L.keys);
  hipLaunchKernelGGL(block_select_kernel, dim3((unsigned)((gq + 3) / 4)), dim3(256), 0, stream, L.keys, gq, L.nqb,
                     L.nkb, L.causal, L.pct, L.kmax, L.idx, L.cnt);
  return hipGetLastError();
}

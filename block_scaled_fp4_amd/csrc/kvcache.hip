// kvcache.hip -- quantize-on-write append to the sink-aware mixed-precision KV
// cache (ScaleSearch page, Metodologia / ScaleSearchAttention: the first and
// last cache blocks stay in full precision, the rest is NVFP4 with
// ScaleSearch).
//
// Appending n_new tokens (a multiple of 16) to batch b: the recent window
// followed by the new tokens forms a sequence T of n_recent + n_new tokens;
// its first n_new tokens move into the NVFP4 region at mid_len[b] (K in
// blocks of 16 channels per token, V in blocks of 16 tokens per channel,
// ScaleSearch over [-2, 6], no per-tensor scale), the window becomes the last
// n_recent tokens of T, and mid_len[b] grows by n_new.  A batch whose NVFP4
// region has no room is left unchanged and flagged.
//
// When T of one operand and 64 channels fits in LDS (the usual case: a
// window of a few hundred tokens), kv_append_fast_kernel does it all in one
// pass and kv_append_finish_kernel updates mid_len and the flags.  Otherwise,
// two launches, so that nothing is overwritten while it may still be read:
//   1. kv_append_quant_kernel: one workgroup per (batch, kv head, 16-token
//      group): one lane per 16-element block (K: 16 tokens x d/16 blocks; V: d
//      channel blocks), the same block quantizer as fp4_quantize; the same
//      launch copies the new window (last n_recent tokens of T) into the
//      workspace;
//   2. kv_append_commit_kernel: window from the workspace, mid_len and flags.
// Launch 1 also keeps each batch's mid_len in the workspace: every workgroup
// of launch 2 decides on that copy, while one of them updates mid_len.
// With the cache's full-precision copy of the middle (the dual cache of the
// ThriftAttention page, Significado), the quantizing lanes of launch 1 also
// write their tokens unquantized, and one more workgroup per (batch, kv head)
// extends the binary64 key-block sums: one lane per channel adds the moved
// tokens in order (sequential, so the sums equal a one-pass sum over each
// block's tokens).
#include "device_common.h"
#include "fp4_internal.h"
#include "quant_core.h"

namespace fp4dev {

constexpr int kCopyTok = 16;  // window tokens per copying workgroup

struct AppendArgs {
  int64_t Hkv, d, mid_cap;
  int n_recent, n_new, ngroups;  // ngroups = n_new / 16
  int ncopy;                     // window chunks of kCopyTok tokens
  const uint16_t* k_new;         // bf16 [B,Hkv,n_new,d]
  const uint16_t* v_new;
  uint16_t* k_recent;            // bf16 [B,Hkv,n_recent,d]
  uint16_t* v_recent;
  uint8_t *kc, *ks, *vc, *vs;
  int32_t* mid_len;
  int32_t* overflow;             // [B], nullable
  uint16_t* ws_k;                // [B,Hkv,n_recent,d] new window
  uint16_t* ws_v;
  int32_t* snap;                 // [B] mid_len as launch 1 read it
  uint16_t* k_mid;               // bf16 [B,Hkv,mid_cap,d] (nullable: no dual copy)
  uint16_t* v_mid;
  double* k_sum;                 // [B,Hkv,nbc,d]
  int nbc;                       // ceil(mid_cap / kDecSelBlock)
  int nsum;                      // 1 with the dual copy (its sums workgroup), else 0
};

// mid_len as the decode kernel reads it: clamped to [0, mid_cap], multiple of 16.
__device__ __forceinline__ int64_t used_mid(const AppendArgs& A, int64_t b) {
  int64_t m = A.mid_len[b];
  if (m < 0) m = 0;
  if (m > A.mid_cap) m = A.mid_cap;
  return m & ~(int64_t)15;
}

// Token t of the sequence T = recent window ++ new tokens of (batch, kv head) bk.
__device__ __forceinline__ const uint16_t* seq_row(const uint16_t* recent, const uint16_t* fresh, const AppendArgs& A,
                                                   int64_t bk, int64_t t) {
  return t < A.n_recent ? recent + (bk * A.n_recent + t) * A.d : fresh + (bk * A.n_new + (t - A.n_recent)) * A.d;
}

// grid: B*Hkv*(ngroups + ncopy + nsum).  Workgroups (bk, g < ngroups)
// quantize group g; workgroups (bk, ngroups + c) copy window chunk c
// (kCopyTok tokens of the new window) into the workspace; with the dual copy
// workgroup (bk, ngroups + ncopy) extends the key-block sums.
__global__ void __launch_bounds__(256) kv_append_quant_kernel(AppendArgs A) {
  __shared__ float2_t tab[128];
  if (threadIdx.x < 128) tab[threadIdx.x] = kScaleTab.v[threadIdx.x];
  __syncthreads();
  const int64_t gi = blockIdx.x;
  const int per = A.ngroups + A.ncopy + A.nsum;
  const int g = (int)(gi % per);
  const int64_t bk = gi / per;
  const int64_t b = bk / A.Hkv;
  if (g == 0 && bk % A.Hkv == 0 && threadIdx.x == 0) A.snap[b] = A.mid_len[b];
  const int64_t mid = used_mid(A, b);
  if (mid + A.n_new > A.mid_cap) return;  // no room: the batch stays as it is
  const int d = (int)A.d;
  if (g == A.ngroups + A.ncopy) {
    // key-block sums: lane c adds channel c of the moved tokens T[0, n_new)
    const int c = threadIdx.x;
    if (c < d) {
      double* sums = A.k_sum + bk * (int64_t)A.nbc * d + c;
      int64_t j = mid / kDecSelBlock;
      double acc = mid % kDecSelBlock == 0 ? 0.0 : sums[j * d];
      for (int t = 0; t < A.n_new; ++t) {
        if (t > 0 && (mid + t) % kDecSelBlock == 0) {
          sums[j * d] = acc;
          ++j;
          acc = 0.0;
        }
        acc = __dadd_rn(acc, (double)bf16_to_f32(seq_row(A.k_recent, A.k_new, A, bk, t)[c]));
      }
      sums[j * d] = acc;
    }
    return;
  }
  if (g >= A.ngroups) {
    // new window: T[n_new + j] for j in this chunk, 16 bytes per step
    const int64_t per_tok = d / 8;  // 16-byte chunks per token
    const int64_t j0 = (int64_t)(g - A.ngroups) * kCopyTok;
    const int64_t j1 = j0 + kCopyTok < A.n_recent ? j0 + kCopyTok : A.n_recent;
    const int64_t n = (j1 - j0) * per_tok;
    for (int64_t i = threadIdx.x; i < n; i += 256) {
      const int64_t j = j0 + i / per_tok, c = (i % per_tok) * 8;
      const int64_t t = A.n_new + j;
      const uint4_t kw = *reinterpret_cast<const uint4_t*>(seq_row(A.k_recent, A.k_new, A, bk, t) + c);
      const uint4_t vw = *reinterpret_cast<const uint4_t*>(seq_row(A.v_recent, A.v_new, A, bk, t) + c);
      *reinterpret_cast<uint4_t*>(A.ws_k + (bk * A.n_recent + j) * d + c) = kw;
      *reinterpret_cast<uint4_t*>(A.ws_v + (bk * A.n_recent + j) * d + c) = vw;
    }
    return;
  }
  const int t0 = 16 * g;           // first token of the group within T
  const int64_t dst_tok = mid + t0;  // its position in the NVFP4 region
  const int nkb = 16 * (d / 16);     // K blocks: 16 tokens x d/16 channel blocks
  const int tid = threadIdx.x;
  if (tid < nkb) {
    // K: token t0 + tid / (d/16), channels 16 * (tid % (d/16)) .. +16
    const int tk = tid / (d / 16), cb = tid % (d / 16);
    const uint16_t* src = seq_row(A.k_recent, A.k_new, A, bk, t0 + tk) + 16 * cb;
    float y[16];
    load8<uint16_t>(src, y);
    load8<uint16_t>(src + 8, y + 8);
    uint32_t codes[2], scale;
    int off;
    quantize_block(y, 1, -2, 6, tab, codes, scale, off);
    const int64_t row = bk * A.mid_cap + dst_tok + tk;
    *reinterpret_cast<uint2_t*>(A.kc + row * (d / 2) + 8 * cb) = uint2_t{codes[0], codes[1]};
    A.ks[row * (d / 16) + cb] = (uint8_t)scale;
    if (A.k_mid) {
      const uint4_t* s4 = reinterpret_cast<const uint4_t*>(src);
      uint4_t* d4 = reinterpret_cast<uint4_t*>(A.k_mid + row * d + 16 * cb);
      d4[0] = s4[0];
      d4[1] = s4[1];
    }
  } else if (tid < nkb + d) {
    // V: channel c of the 16 tokens
    const int c = tid - nkb;
    float y[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) y[k] = bf16_to_f32(seq_row(A.v_recent, A.v_new, A, bk, t0 + k)[c]);
    uint32_t codes[2], scale;
    int off;
    quantize_block(y, 1, -2, 6, tab, codes, scale, off);
    // token pair (2i, 2i+1) of the group -> byte i of the codes, row (dst_tok/2 + i)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      A.vc[(bk * (A.mid_cap / 2) + dst_tok / 2 + i) * d + c] = (uint8_t)((codes[i >> 2] >> (8 * (i & 3))) & 0xFFu);
    A.vs[(bk * (A.mid_cap / 16) + dst_tok / 16) * d + c] = (uint8_t)scale;
    if (A.v_mid) {
#pragma unroll
      for (int k = 0; k < 16; ++k)
        A.v_mid[(bk * A.mid_cap + dst_tok + k) * d + c] = seq_row(A.v_recent, A.v_new, A, bk, t0 + k)[c];
    }
  }
}

// grid: B*Hkv*max(ncopy, 1).  Window chunk c from the workspace, then (the
// first workgroup of kv head 0 of each batch) mid_len and the flag, all
// decided on the mid_len launch 1 saw.
__global__ void __launch_bounds__(256) kv_append_commit_kernel(AppendArgs A) {
  const int nc = A.ncopy > 0 ? A.ncopy : 1;
  const int chunk = (int)(blockIdx.x % nc);
  const int64_t bk = blockIdx.x / nc;
  const int64_t b = bk / A.Hkv;
  int64_t mid = A.snap[b];
  if (mid < 0) mid = 0;
  if (mid > A.mid_cap) mid = A.mid_cap;
  mid &= ~(int64_t)15;
  const bool room = mid + A.n_new <= A.mid_cap;
  const int d = (int)A.d;
  if (room && A.ncopy > 0) {
    const int64_t j0 = (int64_t)chunk * kCopyTok;
    const int64_t j1 = j0 + kCopyTok < A.n_recent ? j0 + kCopyTok : A.n_recent;
    const int64_t base = (bk * A.n_recent + j0) * d / 8, n = (j1 - j0) * d / 8;
    for (int64_t i = threadIdx.x; i < n; i += 256) {
      reinterpret_cast<uint4_t*>(A.k_recent)[base + i] = reinterpret_cast<const uint4_t*>(A.ws_k)[base + i];
      reinterpret_cast<uint4_t*>(A.v_recent)[base + i] = reinterpret_cast<const uint4_t*>(A.ws_v)[base + i];
    }
  }
  if (bk % A.Hkv == 0 && chunk == 0 && threadIdx.x == 0) {
    if (room) A.mid_len[b] = (int32_t)(mid + A.n_new);
    if (A.overflow) A.overflow[b] = room ? 0 : 1;
  }
}

// ---- one-pass append: the sequence T of one (batch, kv head), one operand
// (K or V) and 64 channels fits in LDS (kFastLds bytes), so a workgroup reads
// T once, quantizes its first n_new tokens from LDS and writes the new window
// back over the old one in place (nothing else reads that window), with no
// workspace round trip.  mid_len is read, never written, here; a second
// launch of one thread per batch then updates it and the flags, so every
// workgroup decides on the same value.
constexpr int kFastCh = 64;              // channels per workgroup
constexpr int kFastLds = 62 * 1024;      // bytes of T staged per workgroup (496 tokens)
constexpr int kFastTok = kFastLds / (kFastCh * 2);

// grid: B*Hkv*2*(d/64): (bk, operand, channel half); block 256.
__global__ void __launch_bounds__(256) kv_append_fast_kernel(AppendArgs A) {
  __shared__ float2_t tab[128];
  __shared__ __align__(16) uint16_t Tl[kFastTok * kFastCh];  // [token][channel of this half]
  if (threadIdx.x < 128) tab[threadIdx.x] = kScaleTab.v[threadIdx.x];
  const int nh = (int)(A.d / kFastCh);
  const int64_t gi = blockIdx.x;
  const int half = (int)(gi % nh);
  const bool isv = (gi / nh) % 2 == 1;
  const int64_t bk = gi / (2 * nh), b = bk / A.Hkv;
  const int64_t mid = used_mid(A, b);
  if (mid + A.n_new > A.mid_cap) return;  // no room: the batch stays as it is
  const int d = (int)A.d, c0 = half * kFastCh;
  const int nt = A.n_recent + A.n_new;
  const uint16_t* recent = isv ? A.v_recent : A.k_recent;
  const uint16_t* fresh = isv ? A.v_new : A.k_new;
  // T into LDS: 8 channels (16 bytes) per step
  for (int i = threadIdx.x; i < nt * (kFastCh / 8); i += 256) {
    const int t = i / (kFastCh / 8), c8 = (i % (kFastCh / 8)) * 8;
    *reinterpret_cast<uint4_t*>(Tl + t * kFastCh + c8) =
        *reinterpret_cast<const uint4_t*>(seq_row(recent, fresh, A, bk, t) + c0 + c8);
  }
  __syncthreads();
  // the first n_new tokens of T into the NVFP4 region at mid
  if (!isv) {
    // K: token t, channels 16 cb .. +16 of this half
    for (int i = threadIdx.x; i < A.n_new * (kFastCh / 16); i += 256) {
      const int t = i / (kFastCh / 16), cb = i % (kFastCh / 16);
      float y[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) y[e] = bf16_to_f32(Tl[t * kFastCh + 16 * cb + e]);
      uint32_t codes[2], scale;
      int off;
      quantize_block(y, 1, -2, 6, tab, codes, scale, off);
      const int64_t row = bk * A.mid_cap + mid + t;
      const int gcb = c0 / 16 + cb;
      *reinterpret_cast<uint2_t*>(A.kc + row * (d / 2) + 8 * gcb) = uint2_t{codes[0], codes[1]};
      A.ks[row * (d / 16) + gcb] = (uint8_t)scale;
      if (A.k_mid) {
        const uint4_t* s4 = reinterpret_cast<const uint4_t*>(Tl + t * kFastCh + 16 * cb);
        uint4_t* d4 = reinterpret_cast<uint4_t*>(A.k_mid + row * d + c0 + 16 * cb);
        d4[0] = s4[0];
        d4[1] = s4[1];
      }
    }
  } else {
    // V: channel c of a group of 16 tokens
    for (int i = threadIdx.x; i < (A.n_new / 16) * kFastCh; i += 256) {
      const int g = i / kFastCh, c = i % kFastCh;
      float y[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) y[k] = bf16_to_f32(Tl[(16 * g + k) * kFastCh + c]);
      uint32_t codes[2], scale;
      int off;
      quantize_block(y, 1, -2, 6, tab, codes, scale, off);
      const int64_t tok = mid + 16 * g;
#pragma unroll
      for (int p = 0; p < 8; ++p)
        A.vc[(bk * (A.mid_cap / 2) + tok / 2 + p) * d + c0 + c] = (uint8_t)((codes[p >> 2] >> (8 * (p & 3))) & 0xFFu);
      A.vs[(bk * (A.mid_cap / 16) + tok / 16) * d + c0 + c] = (uint8_t)scale;
      if (A.v_mid) {
#pragma unroll
        for (int k = 0; k < 16; ++k) A.v_mid[(bk * A.mid_cap + tok + k) * d + c0 + c] = Tl[(16 * g + k) * kFastCh + c];
      }
    }
  }
  // the new window: T[n_new + j], j < n_recent, over the old one
  uint16_t* win = isv ? A.v_recent : A.k_recent;
  for (int i = threadIdx.x; i < A.n_recent * (kFastCh / 8); i += 256) {
    const int j = i / (kFastCh / 8), c8 = (i % (kFastCh / 8)) * 8;
    *reinterpret_cast<uint4_t*>(win + (bk * A.n_recent + j) * d + c0 + c8) =
        *reinterpret_cast<const uint4_t*>(Tl + (A.n_new + j) * kFastCh + c8);
  }
  // key-block sums of the moved tokens (K side with the full-precision copy):
  // channel c in token order, a block's sum restarting at its first token
  if (!isv && A.k_mid && threadIdx.x < kFastCh) {
    const int c = threadIdx.x;
    double* sums = A.k_sum + bk * (int64_t)A.nbc * d + c0 + c;
    int64_t j = mid / kDecSelBlock;
    double acc = mid % kDecSelBlock == 0 ? 0.0 : sums[j * d];
    for (int t = 0; t < A.n_new; ++t) {
      if (t > 0 && (mid + t) % kDecSelBlock == 0) {
        sums[j * d] = acc;
        ++j;
        acc = 0.0;
      }
      acc = __dadd_rn(acc, (double)bf16_to_f32(Tl[t * kFastCh + c]));
    }
    sums[j * d] = acc;
  }
}

// grid: ceil(B/256); one thread per batch: mid_len and the flag, decided on
// the mid_len the fast kernel read (it does not write it).
__global__ void __launch_bounds__(256) kv_append_finish_kernel(AppendArgs A, int64_t B) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int64_t mid = used_mid(A, b);
  const bool room = mid + A.n_new <= A.mid_cap;
  if (room) A.mid_len[b] = (int32_t)(mid + A.n_new);
  if (A.overflow) A.overflow[b] = room ? 0 : 1;
}

// grid: B*Hkv*nbc; block: d lanes, one channel each.  Block j's sum over its
// tokens below mid_len, ascending (0 for a block with none).
__global__ void __launch_bounds__(128) kv_block_sums_kernel(const uint16_t* k_mid, const int32_t* mid_len,
                                                            double* k_sum, int64_t Hkv, int64_t mid_cap, int d,
                                                            int nbc) {
  const int64_t gi = blockIdx.x;
  const int64_t bk = gi / nbc;
  const int j = (int)(gi % nbc);
  const int c = threadIdx.x;
  if (c >= d) return;
  int64_t M = mid_len[bk / Hkv];
  if (M < 0) M = 0;
  if (M > mid_cap) M = mid_cap;
  M &= ~(int64_t)15;
  const int64_t t0 = (int64_t)j * kDecSelBlock;
  int64_t n = M - t0;
  if (n < 0) n = 0;
  if (n > kDecSelBlock) n = kDecSelBlock;
  const uint16_t* p = k_mid + (bk * mid_cap + t0) * d + c;
  double s = 0.0;
  int64_t t = 0;
  for (; t + 8 <= n; t += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (double)bf16_to_f32(p[(t + u) * d]);
#pragma unroll
    for (int u = 0; u < 8; ++u) s = __dadd_rn(s, v[u]);
  }
  for (; t < n; ++t) s = __dadd_rn(s, (double)bf16_to_f32(p[t * d]));
  k_sum[(bk * nbc + j) * d + c] = s;
}

}  // namespace fp4dev

using namespace fp4dev;

hipError_t fp4i_launch_kv_block_sums(const void* k_mid, const int32_t* mid_len, double* k_sum, int64_t B,
                                     int64_t Hkv, int64_t mid_cap, int64_t d, hipStream_t st) {
  const int nbc = (int)((mid_cap + kDecSelBlock - 1) / kDecSelBlock);
  if (nbc == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_block_sums_kernel, dim3((unsigned)(B * Hkv * nbc)), dim3(128), 0, st,
                     (const uint16_t*)k_mid, mid_len, k_sum, Hkv, mid_cap, (int)d, nbc);
  return hipGetLastError();
}

size_t fp4i_kv_append_workspace(int64_t B, int64_t Hkv, int64_t n_recent, int64_t d) {
  const size_t win = (size_t)(B * Hkv * n_recent * d) * 2;  // bf16 bytes of one window copy
  const size_t a = (win + 255) & ~(size_t)255;
  return 2 * a + (((size_t)B * 4 + 255) & ~(size_t)255);
}

hipError_t fp4i_launch_kv_append(const KvAppendLaunch& L, hipStream_t st) {
  AppendArgs A;
  A.Hkv = L.Hkv;
  A.d = L.d;
  A.mid_cap = L.mid_cap;
  A.n_recent = L.n_recent;
  A.n_new = L.n_new;
  A.ngroups = L.n_new / 16;
  A.ncopy = (L.n_recent + kCopyTok - 1) / kCopyTok;
  A.k_new = (const uint16_t*)L.k_new;
  A.v_new = (const uint16_t*)L.v_new;
  A.k_recent = (uint16_t*)L.k_recent;
  A.v_recent = (uint16_t*)L.v_recent;
  A.kc = L.kc; A.ks = L.ks; A.vc = L.vc; A.vs = L.vs;
  A.mid_len = L.mid_len;
  A.overflow = L.overflow;
  const size_t win = (size_t)(L.B * L.Hkv * L.n_recent * L.d) * 2;
  const size_t a = (win + 255) & ~(size_t)255;
  A.ws_k = (uint16_t*)L.ws;
  A.ws_v = (uint16_t*)((char*)L.ws + a);
  A.snap = (int32_t*)((char*)L.ws + 2 * a);
  A.k_mid = (uint16_t*)L.k_mid;
  A.v_mid = (uint16_t*)L.v_mid;
  A.k_sum = L.k_sum;
  A.nbc = (int)((L.mid_cap + kDecSelBlock - 1) / kDecSelBlock);
  A.nsum = L.k_mid ? 1 : 0;
  if (L.n_recent + L.n_new <= kFastTok && L.d % kFastCh == 0) {
    const int nh = (int)(L.d / kFastCh);
    hipLaunchKernelGGL(kv_append_fast_kernel, dim3((unsigned)(L.B * L.Hkv * 2 * nh)), dim3(256), 0, st, A);
    hipLaunchKernelGGL(kv_append_finish_kernel, dim3((unsigned)((L.B + 255) / 256)), dim3(256), 0, st, A, L.B);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(kv_append_quant_kernel, dim3((unsigned)(L.B * L.Hkv * (A.ngroups + A.ncopy + A.nsum))), dim3(256),
                     0, st, A);
  const int nc = A.ncopy > 0 ? A.ncopy : 1;
  hipLaunchKernelGGL(kv_append_commit_kernel, dim3((unsigned)(L.B * L.Hkv * nc)), dim3(256), 0, st, A);
  return hipGetLastError();
}

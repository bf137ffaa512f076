// noalloc.hip -- decode for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the decode
// workspace lives in a fixed device array of this library instead of caller
// memory.  Same kernels and results as fp4_attention_decode.
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never uses the array's name as an address: the
// device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept.  Every call on a
// GPU shares that GPU's copy: calls that overlap on one GPU (two streams, two
// threads) race on it.  The decode writes every partial it later reads, so
// nothing has to start at zero.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/fp4.h"
#include "fp4_internal.h"

static __device__ __align__(256) unsigned char scratch[FP4_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch copy (looked up on its first
// use on that device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fp4i_fail(FP4_ERR_HIP, "fp4_attention_decode_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return fp4i_fail(FP4_ERR_UNSUPPORTED, "fp4_attention_decode_noalloc: device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fp4i_fail(FP4_ERR_HIP, "fp4_attention_decode_noalloc: hipGetSymbolAddress(scratch) failed");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FP4_OK;
}

}  // namespace

extern "C" int fp4_attention_decode_noalloc(const void* q, int64_t Hq, const fp4_kv_cache* cache,
                                            float softmax_scale, int32_t out_dtype, void* out, float* lse,
                                            void* stream) {
  const size_t need = fp4_attention_decode_workspace_size(Hq, cache);
  if (need > (size_t)FP4_NOALLOC_SCRATCH_BYTES) {
    char msg[200];
    std::snprintf(msg, sizeof(msg),
                  "fp4_attention_decode_noalloc: needs %zu bytes of scratch, more than the %zu it holds",
                  need, (size_t)FP4_NOALLOC_SCRATCH_BYTES);
    return fp4i_fail(FP4_ERR_UNSUPPORTED, msg);
  }
  // (need == 0: the arguments are invalid; the decode call reports why)
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_address(&ws);
    if (st != FP4_OK) return st;
  }
  return fp4_attention_decode(q, Hq, cache, softmax_scale, out_dtype, out, lse, ws,
                              need > 0 ? (size_t)FP4_NOALLOC_SCRATCH_BYTES : 0, stream);
}

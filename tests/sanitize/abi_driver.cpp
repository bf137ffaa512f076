// Exercises the library's host side -- argument validation and workspace
// sizing of every entry point -- without a GPU; built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_sanitizers.py.  Only calls that
// fail validation or only size workspaces are made, so nothing is launched.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "fp4.h"

#define CHECK(c)                                                    \
  do {                                                              \
    if (!(c)) {                                                     \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                     \
    }                                                               \
  } while (0)

int main() {
  void* f = reinterpret_cast<void*>(uintptr_t(1) << 20);  // never dereferenced
  uint8_t* fb = static_cast<uint8_t*>(f);
  // quantizer
  fp4_quant_opts qo{};
  qo.struct_size = sizeof(qo);
  qo.scale_search = 1;
  qo.f_min = -2;
  qo.f_max = 6;
  CHECK(fp4_quantize(f, FP4_BF16, 16, 40, 40, &qo, fb, fb, nullptr, nullptr, nullptr, 0, nullptr) == FP4_ERR_INVALID_ARG);
  CHECK(std::strlen(fp4_last_error()) > 0);
  CHECK(fp4_quantize(f, 9, 16, 32, 32, &qo, fb, fb, nullptr, nullptr, nullptr, 0, nullptr) == FP4_ERR_INVALID_ARG);
  qo.global_scale = FP4_GLOBAL_AMAX;
  const size_t qws = fp4_quantize_workspace_size(4096, 128, &qo);
  CHECK(qws > 0);
  CHECK(fp4_quantize(f, FP4_BF16, 4096, 128, 128, &qo, fb, fb, nullptr, static_cast<float*>(f), f, qws - 1,
                     nullptr) == FP4_ERR_WORKSPACE);
  qo.hadamard = 1;
  CHECK(fp4_quantize(f, FP4_BF16, 32, 128, 128, &qo, fb, fb, nullptr, static_cast<float*>(f), f, qws,
                     nullptr) == FP4_ERR_INVALID_ARG);
  CHECK(fp4_mx_quantize(f, FP4_BF16, 16, 48, 48, 0, fb, fb, nullptr) == FP4_ERR_INVALID_ARG);
  CHECK(fp4_quantize(nullptr, FP4_BF16, 16, 32, 32, nullptr, fb, fb, nullptr, nullptr, nullptr, 0, nullptr) ==
        FP4_ERR_INVALID_ARG);
  // attention forward, selection, MX, training
  fp4_attn_problem p{};
  p.struct_size = sizeof(p);
  p.B = 1; p.H = 4; p.Hkv = 2; p.Sq = 1000; p.Sk = 1024; p.d = 128;
  p.dtype = FP4_BF16;
  p.q = p.k = p.v = f;
  fp4_attn_opts o{};
  o.struct_size = sizeof(o);
  o.kv_tile = 128; o.scale_search = 1; o.f_min = -2; o.f_max = 6;
  o.fp16_budget_pct = 10; o.sel_block = 128; o.out_dtype = FP4_FP32;
  const size_t aws = fp4_attention_fwd_workspace_size(&p, &o);
  CHECK(aws > 0);
  CHECK(fp4_block_topk_workspace_size(&p, &o) > 0);
  CHECK(fp4_attention_fwd_mx_workspace_size(&p, &o) > 0);
  CHECK(fp4_attention_bwd_workspace_size(&p, &o) > 0);
  CHECK(fp4_attention_fwd(&p, &o, f, nullptr, nullptr, nullptr, f, aws - 1, nullptr) == FP4_ERR_WORKSPACE);
  o.causal = 1;
  CHECK(fp4_attention_fwd(&p, &o, f, nullptr, nullptr, nullptr, f, aws, nullptr) == FP4_ERR_INVALID_ARG);
  o.causal = 0;
  p.d = 96;
  CHECK(fp4_attention_fwd(&p, &o, f, nullptr, nullptr, nullptr, f, aws, nullptr) == FP4_ERR_UNSUPPORTED);
  p.d = 128;
  CHECK(fp4_attention_fwd_mx(&p, &o, f, nullptr, f, 1u << 30, nullptr) == FP4_ERR_INVALID_ARG);  // pct > 0
  o.sel_block = 192;
  CHECK(fp4_block_topk(&p, &o, static_cast<int32_t*>(f), static_cast<int32_t*>(f), f, 1u << 30, nullptr) ==
        FP4_ERR_INVALID_ARG);
  o.sel_block = 128;
  CHECK(fp4_attention_fwd_train(&p, &o, f, f, nullptr, f, 1u << 30, nullptr) != FP4_OK);
  CHECK(fp4_attention_fwd(nullptr, &o, f, nullptr, nullptr, nullptr, f, aws, nullptr) == FP4_ERR_INVALID_ARG);
  // decode, selective decode, block sums, cache append
  fp4_kv_cache c{};
  c.struct_size = sizeof(c);
  c.B = 2; c.Hkv = 2; c.d = 128; c.n_sink = 16; c.n_recent = 32; c.mid_cap = 256;
  c.k_sink = c.v_sink = c.k_recent = c.v_recent = f;
  c.k_codes = c.k_scales = c.v_codes = c.v_scales = fb;
  c.mid_len = static_cast<int32_t*>(f);
  c.k_mid = c.v_mid = f;
  c.k_sum = static_cast<double*>(f);
  const size_t dws = fp4_attention_decode_workspace_size(8, &c);
  CHECK(dws > 0);
  const size_t sws = fp4_attention_decode_selective_workspace_size(8, &c, 10);
  CHECK(sws > dws);
  CHECK(fp4_attention_decode(f, 8, &c, 0.0f, FP4_FP32, f, nullptr, f, dws - 1, nullptr) == FP4_ERR_WORKSPACE);
  CHECK(fp4_attention_decode(f, 7, &c, 0.0f, FP4_FP32, f, nullptr, f, dws, nullptr) == FP4_ERR_INVALID_ARG);
  CHECK(fp4_attention_decode_selective(f, 8, &c, 101, 0.0f, FP4_FP32, f, nullptr, nullptr, nullptr, f, sws,
                                       nullptr) == FP4_ERR_INVALID_ARG);
  const size_t kws = fp4_kv_cache_append_workspace_size(&c);
  CHECK(kws > 0);
  CHECK(fp4_kv_cache_append(&c, f, f, 24, nullptr, f, kws, nullptr) == FP4_ERR_INVALID_ARG);
  c.mid_cap = 100;
  CHECK(fp4_kv_block_sums(&c, nullptr) == FP4_ERR_INVALID_ARG);
  CHECK(fp4_version() > 0);
  std::printf("abi driver ok\n");
  return 0;
}

// api.cpp -- extern "C" entry points of the FP4 library: argument validation,
// workspace planning and kernel launches.  No allocation; no synchronization
// unless FP4_SYNC_CHECK is set.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/fp4.h"
#include "fp4_internal.h"

namespace {

thread_local char g_err[512] = "";

// Debug switches read from the environment at every call (set and unset at will):
// FP4_LOG=1 reports each launch and each error on stderr; FP4_SYNC_CHECK=1
// waits for the device after each launch, so a fault inside a kernel is
// returned as FP4_ERR_HIP by the call that launched it.
bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] && std::strcmp(v, "0") != 0;
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  if (env_on("FP4_LOG")) std::fprintf(stderr, "[fp4] error %d: %s\n", code, g_err);
  return code;
}

int ok() {
  g_err[0] = 0;
  return FP4_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Base-2 score factor: log2(e) * scale rounded once to binary32, scale = 1/sqrt(d)
// when the caller passes <= 0.
float score_factor(float softmax_scale, int64_t d) {
  double s = softmax_scale > 0.0f ? (double)softmax_scale : 1.0 / std::sqrt((double)d);
  return (float)(1.4426950408889634074 * s);
}

int check_quant_opts(const fp4_quant_opts* o) {
  if (!o) return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: opts is NULL");
  if (o->struct_size < sizeof(fp4_quant_opts))
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: opts->struct_size %u < %zu", o->struct_size,
                sizeof(fp4_quant_opts));
  if (o->scale_search != 0 && o->scale_search != 1)
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: scale_search must be 0 or 1");
  if (o->scale_search && (o->f_min > 0 || o->f_max < 0 || o->f_min < -8 || o->f_max > 8))
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: need -8 <= f_min <= 0 <= f_max <= 8");
  if (o->global_scale < FP4_GLOBAL_NONE || o->global_scale > FP4_GLOBAL_GIVEN)
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: bad global_scale mode %d", o->global_scale);
  if (o->block_axis != 0 && o->block_axis != 1)
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: block_axis must be 0 or 1");
  if (o->hadamard != 0 && o->hadamard != 1) return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: hadamard must be 0 or 1");
  if (o->hadamard && o->block_axis != 0)
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: hadamard needs block_axis 0");
  if (o->hadamard && o->global_scale == FP4_GLOBAL_AMAX)
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: hadamard with FP4_GLOBAL_AMAX is not supported");
  if (o->channel_exp) {
    if (o->block_axis != 0) return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: channel_exp needs block_axis 0");
    if (o->exp_negate != 0 && o->exp_negate != 1)
      return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: exp_negate must be 0 or 1");
    if (o->exp_rows < 1) return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: exp_rows must be >= 1");
    if (o->global_scale == FP4_GLOBAL_AMAX)
      return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: channel_exp with FP4_GLOBAL_AMAX is not supported");
    if (!aligned16(o->channel_exp)) return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: channel_exp must be 16-byte aligned");
  }
  return FP4_OK;
}

bool hadamard_size(int64_t n) { return n == 16 || n == 32 || n == 64 || n == 128; }

// binary32 1/sqrt(n) for the incoherence rotation, rounded once from binary64
float hadamard_scale(int64_t n) { return (float)(1.0 / std::sqrt((double)n)); }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess && env_on("FP4_SYNC_CHECK")) {
    e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e != hipSuccess) return fail(FP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  if (env_on("FP4_LOG")) std::fprintf(stderr, "[fp4] %s: ok\n", what);
  return ok();
}

struct AttnPlan {
  size_t qc, qs, kc, ks, vc, vs, qm, km, idx, cnt, keys, bpart, bexp, total;
  int nqb, nkb, kmax;
  bool need_quant, need_sel;
};

AttnPlan plan_attn(const fp4_attn_problem* p, const fp4_attn_opts* o) {
  AttnPlan P{};
  const int64_t B = p->B, H = p->H, Hkv = p->Hkv, Sq = p->Sq, Sk = p->Sk, d = p->d;
  P.need_quant = !(p->q_codes && p->q_scales && p->k_codes && p->k_scales && p->v_codes && p->v_scales);
  P.need_sel = o->fp16_budget_pct > 0 && !o->selection_given;
  const int sb = o->sel_block > 0 ? o->sel_block : 128;
  P.nqb = (int)((Sq + sb - 1) / sb);
  P.nkb = (int)((Sk + sb - 1) / sb);
  P.kmax = o->fp16_budget_pct > 0 ? (o->fp16_budget_pct * P.nkb + 99) / 100 : 0;
  size_t off = 0;
  auto take = [&](size_t n) { size_t at = off; off += align256(n); return at; };
  if (P.need_quant) {
    P.qc = take((size_t)(B * H * Sq * d / 2));
    P.qs = take((size_t)(B * H * Sq * d / 16));
    P.kc = take((size_t)(B * Hkv * Sk * d / 2));
    P.ks = take((size_t)(B * Hkv * Sk * d / 16));
    P.vc = take((size_t)(B * Hkv * Sk * d / 2));
    P.vs = take((size_t)(B * Hkv * Sk * d / 16));
    if (o->balance_qk) {
      P.bpart = take(fp4i_balance_partials(B, H, Hkv, Sq, Sk, d) * sizeof(double));
      P.bexp = take((size_t)(B * Hkv * d) * sizeof(int32_t));
    }
  }
  if (P.need_sel) {
    P.qm = take((size_t)(B * H * P.nqb * d) * sizeof(double));
    P.km = take((size_t)(B * Hkv * P.nkb * d) * sizeof(double));
    P.idx = take((size_t)(B * H * P.nqb * (P.kmax > 0 ? P.kmax : 1)) * sizeof(int32_t));
    P.cnt = take((size_t)(B * H * P.nqb) * sizeof(int32_t));
    P.keys = take((size_t)(B * H * P.nqb) * (size_t)P.nkb * sizeof(uint64_t));
  }
  P.total = off;
  return P;
}

// Row maps of q, k and v: the problem's strides, or dense where all three of a
// tensor's strides are zero.
struct Maps {
  TokMap q, k, v;
  bool strided = false;  // some tensor is not dense
};

Maps maps_of(const fp4_attn_problem* p) {
  Maps m;
  m.q = dense_map(p->H, p->Sq, p->d);
  m.k = dense_map(p->Hkv, p->Sk, p->d);
  m.v = dense_map(p->Hkv, p->Sk, p->d);
  auto set = [&](TokMap& t, const int64_t st[3]) {
    if (!st[0] && !st[1] && !st[2]) return;
    if (st[0] != t.bs || st[1] != t.hs || st[2] != t.ts) m.strided = true;
    t.bs = st[0];
    t.hs = st[1];
    t.ts = st[2];
  };
  set(m.q, p->q_strides);
  set(m.k, p->k_strides);
  set(m.v, p->v_strides);
  return m;
}

// Strides of one high-precision input: none, or all three with whole 16-byte
// rows (multiples of 8 elements), token rows at least d apart, and (k, v) one
// head's rows within 32-bit byte offsets.
int check_strides(const int64_t st[3], int64_t S, int64_t d, bool kv, const char* fn, const char* name) {
  if (!st[0] && !st[1] && !st[2]) return FP4_OK;
  if (st[0] < 0 || st[1] < 0 || st[2] < d)
    return fail(FP4_ERR_INVALID_ARG, "%s: %s strides must be >= 0 with the token stride >= d", fn, name);
  if (st[0] % 8 || st[1] % 8 || st[2] % 8)
    return fail(FP4_ERR_INVALID_ARG, "%s: %s strides must be multiples of 8 elements (16-byte rows)", fn, name);
  if (kv && ((S - 1) * st[2] + d) * 2 >= ((int64_t)1 << 31))
    return fail(FP4_ERR_UNSUPPORTED, "%s: %s token stride too large for one head's 32-bit offsets", fn, name);
  return FP4_OK;
}

int check_attn(const fp4_attn_problem* p, const fp4_attn_opts* o, const char* fn, bool for_topk) {
  if (!p || !o) return fail(FP4_ERR_INVALID_ARG, "%s: problem or opts is NULL", fn);
  if (p->struct_size < sizeof(fp4_attn_problem) || o->struct_size < sizeof(fp4_attn_opts))
    return fail(FP4_ERR_INVALID_ARG, "%s: struct_size too small", fn);
  if (p->B < 1 || p->H < 1 || p->Hkv < 1 || p->Sq < 1 || p->Sk < 1)
    return fail(FP4_ERR_INVALID_ARG, "%s: B, H, Hkv, Sq, Sk must be >= 1", fn);
  if (p->H % p->Hkv) return fail(FP4_ERR_INVALID_ARG, "%s: H %% Hkv != 0", fn);
  if (p->d != 64 && p->d != 128) return fail(FP4_ERR_UNSUPPORTED, "%s: head dim %lld not in {64,128}", fn, (long long)p->d);
  if (p->Sk % 16) return fail(FP4_ERR_INVALID_ARG, "%s: Sk %% 16 != 0", fn);
  // kernels address one head's K/V through 32-bit buffer offsets
  if (p->Sk * p->d * 2 >= ((int64_t)1 << 31)) return fail(FP4_ERR_UNSUPPORTED, "%s: Sk * d too large", fn);
  if (p->dtype != FP4_BF16 && p->dtype != FP4_FP16)
    return fail(FP4_ERR_UNSUPPORTED, "%s: q/k/v dtype must be bf16 or fp16", fn);
  if (o->causal != 0 && o->causal != 1) return fail(FP4_ERR_INVALID_ARG, "%s: causal must be 0 or 1", fn);
  if (o->causal && p->Sq != p->Sk) return fail(FP4_ERR_INVALID_ARG, "%s: causal needs Sq == Sk", fn);
  if (o->kv_tile != 64 && o->kv_tile != 128) return fail(FP4_ERR_UNSUPPORTED, "%s: kv_tile must be 64 or 128", fn);
  if (o->fp16_budget_pct < 0 || o->fp16_budget_pct > 100)
    return fail(FP4_ERR_INVALID_ARG, "%s: fp16_budget_pct must be in [0,100]", fn);
  // a selection block holds whole 128-row query tiles of the kernel and whole key tiles
  if (o->fp16_budget_pct > 0 && (o->sel_block <= 0 || o->sel_block % 128 || o->sel_block % o->kv_tile ||
                                 o->sel_block > 4096))
    return fail(FP4_ERR_INVALID_ARG, "%s: sel_block must be a positive multiple of 128 (<= 4096)", fn);
  if (o->fp16_budget_pct > 0 && (p->Sk + o->sel_block - 1) / o->sel_block > 4096)
    return fail(FP4_ERR_UNSUPPORTED, "%s: more than 4096 key blocks", fn);
  if (o->fp16_budget_pct > 0 && (!p->q || !p->k || !p->v))
    return fail(FP4_ERR_INVALID_ARG, "%s: the FP16 path needs the high-precision q, k, v", fn);
  if (for_topk && o->fp16_budget_pct == 0) return fail(FP4_ERR_INVALID_ARG, "%s: fp16_budget_pct is 0", fn);
  if (o->selection_given != 0 && o->selection_given != 1)
    return fail(FP4_ERR_INVALID_ARG, "%s: selection_given must be 0 or 1", fn);
  if (o->scale_search != 0 && o->scale_search != 1) return fail(FP4_ERR_INVALID_ARG, "%s: scale_search must be 0 or 1", fn);
  if (o->scale_search && (o->f_min > 0 || o->f_max < 0 || o->f_min < -8 || o->f_max > 8))
    return fail(FP4_ERR_INVALID_ARG, "%s: need -8 <= f_min <= 0 <= f_max <= 8", fn);
  if (o->out_dtype < FP4_BF16 || o->out_dtype > FP4_FP32) return fail(FP4_ERR_INVALID_ARG, "%s: bad out_dtype", fn);
  const bool any_codes = p->q_codes || p->q_scales || p->k_codes || p->k_scales || p->v_codes || p->v_scales;
  const bool all_codes = p->q_codes && p->q_scales && p->k_codes && p->k_scales && p->v_codes && p->v_scales;
  if (any_codes && !all_codes) return fail(FP4_ERR_INVALID_ARG, "%s: give all six quantized arrays or none", fn);
  if (!all_codes && (!p->q || !p->k || !p->v)) return fail(FP4_ERR_INVALID_ARG, "%s: q, k, v are NULL", fn);
  if (o->hadamard_qk != 0 && o->hadamard_qk != 1) return fail(FP4_ERR_INVALID_ARG, "%s: hadamard_qk must be 0 or 1", fn);
  if (o->p_single_level != 0 && o->p_single_level != 1)
    return fail(FP4_ERR_INVALID_ARG, "%s: p_single_level must be 0 or 1", fn);
  if (o->hadamard_qk && all_codes)
    return fail(FP4_ERR_INVALID_ARG, "%s: hadamard_qk applies to the call's own quantization (no pre-quantized operands)", fn);
  if (o->balance_qk != 0 && o->balance_qk != 1) return fail(FP4_ERR_INVALID_ARG, "%s: balance_qk must be 0 or 1", fn);
  if (o->balance_qk && all_codes)
    return fail(FP4_ERR_INVALID_ARG, "%s: balance_qk applies to the call's own quantization (no pre-quantized operands)", fn);
  const void* ptrs[] = {p->q, p->k, p->v, p->q_codes, p->q_scales, p->k_codes, p->k_scales, p->v_codes, p->v_scales};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(FP4_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  int st = check_strides(p->q_strides, p->Sq, p->d, false, fn, "q");
  if (!st) st = check_strides(p->k_strides, p->Sk, p->d, true, fn, "k");
  if (!st) st = check_strides(p->v_strides, p->Sk, p->d, true, fn, "v");
  return st;
}

}  // namespace

// Error reporting for the library's other host sources (same message buffer).
int fp4i_fail(int code, const char* msg) { return fail(code, "%s", msg); }

extern "C" {

int fp4_version(void) { return 10000; }

const char* fp4_last_error(void) { return g_err; }

size_t fp4_quantize_workspace_size(int64_t rows, int64_t cols, const fp4_quant_opts* opts) {
  if (!opts || opts->global_scale != FP4_GLOBAL_AMAX || rows <= 0 || cols <= 0) return 0;
  return (size_t)fp4i_amax_parts(rows, cols) * sizeof(float);
}

int fp4_quantize(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                 const fp4_quant_opts* opts, uint8_t* codes, uint8_t* scales, int8_t* offsets,
                 float* g, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_quant_opts(opts);
  if (st) return st;
  if (dtype != FP4_BF16 && dtype != FP4_FP16 && dtype != FP4_FP32)
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: bad dtype %d", dtype);
  if (rows < 0 || cols < 0 || ld < cols) return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: bad shape/ld");
  if (opts->block_axis == 0 && cols % 16) return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: cols %% 16 != 0");
  if (opts->block_axis == 1 && rows % 16) return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: rows %% 16 != 0");
  if (opts->channel_exp && rows % opts->exp_rows)
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: exp_rows must divide rows");
  if (opts->hadamard && !hadamard_size(cols))
    return fail(FP4_ERR_UNSUPPORTED, "fp4_quantize: hadamard needs cols in {16, 32, 64, 128}");
  if (rows > 0 && cols > 0 && (!x || !codes || !scales))
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: x, codes and scales must be non-NULL");
  if ((x && !aligned16(x)) || (codes && !aligned16(codes)) || (scales && !aligned16(scales)))
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: x, codes, scales must be 16-byte aligned");
  const size_t esz = dtype == FP4_FP32 ? 4 : 2;
  if (opts->block_axis == 0 && ld > cols && ((ld * esz) % 16))
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: row stride must keep 16-byte alignment");
  if (opts->global_scale != FP4_GLOBAL_NONE && !g)
    return fail(FP4_ERR_INVALID_ARG, "fp4_quantize: g is required for this global_scale mode");
  const size_t need = fp4_quantize_workspace_size(rows, cols, opts);
  if (workspace_bytes < need || (need && !workspace))
    return fail(FP4_ERR_WORKSPACE, "fp4_quantize: workspace needs %zu bytes", need);
  QuantLaunch L{};
  L.x = x;
  L.dtype = dtype;
  L.rows = rows;
  L.cols = cols;
  L.ld = ld;
  L.axis = opts->block_axis;
  L.search = opts->scale_search;
  L.fmin = opts->f_min;
  L.fmax = opts->f_max;
  L.gmode = opts->global_scale;
  L.codes = codes;
  L.scales = scales;
  L.offsets = offsets;
  L.g = g;
  L.amax_ws = (float*)workspace;
  L.hadamard = opts->hadamard;
  for (int i = 0; i < 4; ++i) L.hsigns[i] = opts->hadamard_signs[i];
  L.hscale = hadamard_scale(cols);
  L.cexp = opts->channel_exp;
  L.exp_negate = opts->exp_negate;
  L.exp_rows = opts->exp_rows;
  return hip_status(fp4i_launch_quantize(L, (hipStream_t)stream), "fp4_quantize launch");
}

int fp4_mx_quantize(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld, int32_t block_axis,
                    uint8_t* codes, uint8_t* scales, void* stream) {
  const char* fn = "fp4_mx_quantize";
  if (dtype != FP4_BF16 && dtype != FP4_FP16 && dtype != FP4_FP32) return fail(FP4_ERR_INVALID_ARG, "%s: bad dtype", fn);
  if (block_axis != 0 && block_axis != 1) return fail(FP4_ERR_INVALID_ARG, "%s: block_axis must be 0 or 1", fn);
  if (rows < 0 || cols < 0 || ld < cols) return fail(FP4_ERR_INVALID_ARG, "%s: bad shape/ld", fn);
  if (block_axis == 0 && cols % 32) return fail(FP4_ERR_INVALID_ARG, "%s: cols %% 32 != 0", fn);
  if (block_axis == 1 && rows % 32) return fail(FP4_ERR_INVALID_ARG, "%s: rows %% 32 != 0", fn);
  if (rows > 0 && cols > 0 && (!x || !codes || !scales)) return fail(FP4_ERR_INVALID_ARG, "%s: x, codes, scales required", fn);
  if ((x && !aligned16(x)) || (codes && !aligned16(codes)))
    return fail(FP4_ERR_INVALID_ARG, "%s: x and codes must be 16-byte aligned", fn);
  const size_t esz = dtype == FP4_FP32 ? 4 : 2;
  if (block_axis == 0 && ld > cols && ((ld * esz) % 16)) return fail(FP4_ERR_INVALID_ARG, "%s: row stride must keep 16-byte alignment", fn);
  return hip_status(fp4i_launch_mx_quantize(x, dtype, rows, cols, ld, block_axis, codes, scales, (hipStream_t)stream),
                    "fp4_mx_quantize launch");
}

size_t fp4_attention_fwd_workspace_size(const fp4_attn_problem* prob, const fp4_attn_opts* opts) {
  if (!prob || !opts || prob->struct_size < sizeof(fp4_attn_problem) || opts->struct_size < sizeof(fp4_attn_opts))
    return 0;
  return plan_attn(prob, opts).total;
}

size_t fp4_block_topk_workspace_size(const fp4_attn_problem* prob, const fp4_attn_opts* opts) {
  if (!prob || !opts || prob->struct_size < sizeof(fp4_attn_problem) || opts->struct_size < sizeof(fp4_attn_opts))
    return 0;
  fp4_attn_opts o2 = *opts;
  o2.selection_given = 0;
  AttnPlan P = plan_attn(prob, &o2);
  if (!P.need_sel) return 0;
  return P.total - P.qm;  // the selection part only
}

static int launch_selection(const fp4_attn_problem* p, const fp4_attn_opts* o, const AttnPlan& P, char* ws_sel,
                            int32_t* idx, int32_t* cnt, hipStream_t s, bool means_ready = false) {
  TopkLaunch T;
  T.means_ready = means_ready ? 1 : 0;
  T.q = p->q;
  T.k = p->k;
  T.dtype = p->dtype;
  T.B = p->B; T.H = p->H; T.Hkv = p->Hkv; T.Sq = p->Sq; T.Sk = p->Sk; T.d = p->d;
  T.causal = o->causal;
  T.pct = o->fp16_budget_pct;
  T.sel_block = o->sel_block;
  T.nqb = P.nqb; T.nkb = P.nkb; T.kmax = P.kmax;
  const Maps m = maps_of(p);
  T.qmap = m.q;
  T.kmap = m.k;
  T.qmeans = (double*)(ws_sel);
  T.kmeans = (double*)(ws_sel + (P.km - P.qm));
  T.idx = idx ? idx : (int32_t*)(ws_sel + (P.idx - P.qm));
  T.cnt = cnt ? cnt : (int32_t*)(ws_sel + (P.cnt - P.qm));
  T.keys = (uint64_t*)(ws_sel + (P.keys - P.qm));
  return hip_status(fp4i_launch_topk(T, s), "block selection launch");
}

size_t fp4_qk_balance_workspace_size(const fp4_attn_problem* prob) {
  if (!prob || prob->struct_size < sizeof(fp4_attn_problem) || prob->B < 1 || prob->H < 1 || prob->Hkv < 1 ||
      prob->Sq < 1 || prob->Sk < 1 || prob->H % prob->Hkv || (prob->d != 64 && prob->d != 128))
    return 0;
  return fp4i_balance_partials(prob->B, prob->H, prob->Hkv, prob->Sq, prob->Sk, prob->d) * sizeof(double);
}

int fp4_qk_balance(const fp4_attn_problem* prob, int32_t* exponents, void* workspace, size_t workspace_bytes,
                   void* stream) {
  const char* fn = "fp4_qk_balance";
  if (!prob || prob->struct_size < sizeof(fp4_attn_problem)) return fail(FP4_ERR_INVALID_ARG, "%s: bad problem", fn);
  if (prob->B < 1 || prob->H < 1 || prob->Hkv < 1 || prob->Sq < 1 || prob->Sk < 1 || prob->H % prob->Hkv)
    return fail(FP4_ERR_INVALID_ARG, "%s: bad B/H/Hkv/Sq/Sk", fn);
  if (prob->d != 64 && prob->d != 128) return fail(FP4_ERR_UNSUPPORTED, "%s: head dim must be 64 or 128", fn);
  if (prob->dtype != FP4_BF16 && prob->dtype != FP4_FP16) return fail(FP4_ERR_UNSUPPORTED, "%s: bf16 or fp16", fn);
  if (!prob->q || !prob->k || !exponents) return fail(FP4_ERR_INVALID_ARG, "%s: q, k and exponents are required", fn);
  if (!aligned16(prob->q) || !aligned16(prob->k)) return fail(FP4_ERR_INVALID_ARG, "%s: q, k must be 16-byte aligned", fn);
  const size_t need = fp4_qk_balance_workspace_size(prob);
  if (workspace_bytes < need || !workspace) return fail(FP4_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  int st = check_strides(prob->q_strides, prob->Sq, prob->d, false, fn, "q");
  if (!st) st = check_strides(prob->k_strides, prob->Sk, prob->d, true, fn, "k");
  if (st) return st;
  const Maps m = maps_of(prob);
  BalanceLaunch BL{};
  BL.q = prob->q; BL.k = prob->k; BL.dtype = prob->dtype;
  BL.B = prob->B; BL.H = prob->H; BL.Hkv = prob->Hkv; BL.Sq = prob->Sq; BL.Sk = prob->Sk; BL.d = prob->d;
  BL.qmap = m.q; BL.kmap = m.k;
  BL.partial = (double*)workspace;
  BL.exps = exponents;
  return hip_status(fp4i_launch_balance(BL, (hipStream_t)stream), "fp4_qk_balance launch");
}

int fp4_block_topk(const fp4_attn_problem* prob, const fp4_attn_opts* opts, int32_t* topk_idx,
                   int32_t* topk_cnt, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_attn(prob, opts, "fp4_block_topk", true);
  if (st) return st;
  if (!prob->q || !prob->k) return fail(FP4_ERR_INVALID_ARG, "fp4_block_topk: q and k are required");
  fp4_attn_opts o2 = *opts;
  o2.selection_given = 0;
  AttnPlan P = plan_attn(prob, &o2);
  size_t need = P.total - P.qm;
  if (workspace_bytes < need || !workspace) return fail(FP4_ERR_WORKSPACE, "fp4_block_topk: workspace needs %zu bytes", need);
  if (!topk_idx || !topk_cnt) return fail(FP4_ERR_INVALID_ARG, "fp4_block_topk: topk_idx and topk_cnt are required");
  return launch_selection(prob, opts, P, (char*)workspace, topk_idx, topk_cnt, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// The forward: quantization and selection into the workspace when needed, then
// the attention kernel for `out`, and with out_hp the same kernel with
// unquantized P on the FP4 tiles for the high-precision output.
int attention_fwd_impl(const fp4_attn_problem* prob, const fp4_attn_opts* opts, void* out, void* out_hp,
                       float* lse, int32_t* topk_idx, int32_t* topk_cnt, void* workspace, size_t workspace_bytes,
                       void* stream) {
  AttnPlan P = plan_attn(prob, opts);
  if (workspace_bytes < P.total || (P.total && !workspace))
    return fail(FP4_ERR_WORKSPACE, "fp4_attention_fwd: workspace needs %zu bytes", P.total);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int64_t B = prob->B, H = prob->H, Hkv = prob->Hkv, Sq = prob->Sq, Sk = prob->Sk, d = prob->d;
  const uint8_t *qc = prob->q_codes, *qs = prob->q_scales, *kc = prob->k_codes, *ks = prob->k_scales,
                *vc = prob->v_codes, *vs = prob->v_scales;
  const Maps maps = maps_of(prob);
  if (P.need_quant) {
    QuantLaunch L{};
    L.dtype = prob->dtype;
    L.search = opts->scale_search;
    L.fmin = opts->f_min;
    L.fmax = opts->f_max;
    L.gmode = 0;
    L.cols = d;
    L.ld = d;
    L.strided = maps.strided ? 1 : 0;
    L.map = maps.q;
    L.x = prob->q; L.rows = B * H * Sq; L.axis = 0;
    L.codes = (uint8_t*)(ws + P.qc); L.scales = (uint8_t*)(ws + P.qs);
    L.hadamard = opts->hadamard_qk;  // Q and K only; V is never rotated
    for (int i = 0; i < 4; ++i) L.hsigns[i] = opts->hadamard_signs[i];
    L.hscale = hadamard_scale(d);
    hipError_t e = hipSuccess;
    if (opts->balance_qk) {  // exponents of the pair Q 2^-e, K 2^e, applied by the row quantizer
      BalanceLaunch BL{};
      BL.q = prob->q; BL.k = prob->k; BL.dtype = prob->dtype;
      BL.B = B; BL.H = H; BL.Hkv = Hkv; BL.Sq = Sq; BL.Sk = Sk; BL.d = d;
      BL.qmap = maps.q; BL.kmap = maps.k;
      BL.partial = (double*)(ws + P.bpart);
      BL.exps = (int32_t*)(ws + P.bexp);
      e = fp4i_launch_balance(BL, s);
      L.cexp = BL.exps;
      L.exp_negate = 1;
      L.exp_rows = (H / Hkv) * Sq;  // the query heads of a kv head are consecutive
    }
    // with the selection computed here, the Q and K launches also write the
    // selection's block means (from the unrotated, unbalanced input)
    if (P.need_sel) {
      L.means = (double*)(ws + P.qm);
      L.mS = Sq;
      L.mblk = opts->sel_block;
      L.mnb = P.nqb;
    }
    QuantLaunch LK = L;
    LK.x = prob->k; LK.rows = B * Hkv * Sk;
    LK.map = maps.k;
    LK.codes = (uint8_t*)(ws + P.kc); LK.scales = (uint8_t*)(ws + P.ks);
    LK.exp_negate = 0;
    LK.exp_rows = Sk;
    if (P.need_sel) {
      LK.means = (double*)(ws + P.km);
      LK.mS = Sk;
      LK.mnb = P.nkb;
    }
    QuantLaunch LV = LK;
    LV.x = prob->v; LV.axis = 1; LV.hadamard = 0;  // V blocks run along tokens (16-token blocks never straddle heads: Sk % 16 == 0)
    LV.map = maps.v;
    LV.cexp = nullptr;
    LV.means = nullptr;
    LV.codes = (uint8_t*)(ws + P.vc); LV.scales = (uint8_t*)(ws + P.vs);
    if (e == hipSuccess) {
      // the plain case (no rotation, balance or block means) in one launch
      if (!L.hadamard && !L.cexp && !L.means) {
        e = fp4i_launch_quantize_qkv(L, LK, LV, s);
      } else {
        e = fp4i_launch_quantize(L, s);
        if (e == hipSuccess) e = fp4i_launch_quantize(LK, s);
        if (e == hipSuccess) e = fp4i_launch_quantize(LV, s);
      }
    }
    if (e != hipSuccess) return hip_status(e, "fp4_attention_fwd quantize launch");
    qc = (uint8_t*)(ws + P.qc); qs = (uint8_t*)(ws + P.qs);
    kc = (uint8_t*)(ws + P.kc); ks = (uint8_t*)(ws + P.ks);
    vc = (uint8_t*)(ws + P.vc); vs = (uint8_t*)(ws + P.vs);
  }
  const int32_t* idx = nullptr;
  const int32_t* cnt = nullptr;
  if (opts->fp16_budget_pct > 0 && opts->selection_given) {
    if (!topk_idx || !topk_cnt)
      return fail(FP4_ERR_INVALID_ARG, "fp4_attention_fwd: selection_given needs topk_idx and topk_cnt");
    idx = topk_idx;
    cnt = topk_cnt;
  } else if (P.need_sel) {
    const int st = launch_selection(prob, opts, P, ws + P.qm, topk_idx, topk_cnt, s, P.need_quant);
    if (st) return st;
    idx = topk_idx ? topk_idx : (const int32_t*)(ws + P.idx);
    cnt = topk_cnt ? topk_cnt : (const int32_t*)(ws + P.cnt);
  }
  AttnLaunch A;
  A.B = B; A.H = H; A.Hkv = Hkv; A.Sq = Sq; A.Sk = Sk; A.d = d;
  A.dtype = prob->dtype;
  A.q = prob->q; A.k = prob->k; A.v = prob->v;
  A.qmap = maps.q; A.kmap = maps.k; A.vmap = maps.v;
  A.strided = maps.strided ? 1 : 0;
  A.qc = qc; A.qs = qs; A.kc = kc; A.ks = ks; A.vc = vc; A.vs = vs;
  A.causal = opts->causal;
  A.c = score_factor(opts->softmax_scale, d);
  A.kv_tile = opts->kv_tile;
  A.pct = opts->fp16_budget_pct;
  A.p_mode = opts->p_single_level ? 1 : 0;
  A.sel_block = opts->sel_block;
  A.nqb = P.nqb;
  A.kmax = P.kmax;
  A.idx = idx;
  A.cnt = cnt;
  A.out_dtype = opts->out_dtype;
  A.out = out;
  A.lse = lse;
  const int st2 = hip_status(fp4i_launch_attn_fwd(A, s), "fp4_attention_fwd launch");
  if (st2 || !out_hp) return st2;
  A.p_mode = 2;
  A.out = out_hp;
  A.lse = nullptr;
  return hip_status(fp4i_launch_attn_fwd(A, s), "fp4_attention_fwd_train launch");
}

}  // namespace

extern "C" {

int fp4_attention_fwd(const fp4_attn_problem* prob, const fp4_attn_opts* opts, void* out, float* lse,
                      int32_t* topk_idx, int32_t* topk_cnt, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int st = check_attn(prob, opts, "fp4_attention_fwd", false);
  if (st) return st;
  if (!out || !aligned16(out)) return fail(FP4_ERR_INVALID_ARG, "fp4_attention_fwd: out must be non-NULL and 16-byte aligned");
  return attention_fwd_impl(prob, opts, out, nullptr, lse, topk_idx, topk_cnt, workspace, workspace_bytes, stream);
}

size_t fp4_attention_fwd_mx_workspace_size(const fp4_attn_problem* prob, const fp4_attn_opts* opts) {
  if (!prob || !opts || prob->struct_size < sizeof(fp4_attn_problem) || opts->struct_size < sizeof(fp4_attn_opts))
    return 0;
  if (prob->q_codes && prob->q_scales && prob->k_codes && prob->k_scales && prob->v_codes && prob->v_scales) return 0;
  const size_t nq = (size_t)(prob->B * prob->H * prob->Sq * prob->d), nk = (size_t)(prob->B * prob->Hkv * prob->Sk * prob->d);
  return align256(nq / 2) + align256(nq / 32) + 2 * (align256(nk / 2) + align256(nk / 32));
}

int fp4_attention_fwd_mx(const fp4_attn_problem* prob, const fp4_attn_opts* opts, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "fp4_attention_fwd_mx";
  int st = check_attn(prob, opts, fn, false);
  if (st) return st;
  if (opts->fp16_budget_pct != 0) return fail(FP4_ERR_INVALID_ARG, "%s: no FP16 path (fp16_budget_pct must be 0)", fn);
  if (opts->hadamard_qk) return fail(FP4_ERR_INVALID_ARG, "%s: hadamard_qk must be 0", fn);
  if (opts->balance_qk) return fail(FP4_ERR_INVALID_ARG, "%s: balance_qk must be 0", fn);
  if (prob->Sk % 32) return fail(FP4_ERR_INVALID_ARG, "%s: Sk %% 32 != 0", fn);
  if (maps_of(prob).strided) return fail(FP4_ERR_UNSUPPORTED, "%s: q, k, v must be dense", fn);
  if (!out || !aligned16(out)) return fail(FP4_ERR_INVALID_ARG, "%s: out must be non-NULL and 16-byte aligned", fn);
  const size_t need = fp4_attention_fwd_mx_workspace_size(prob, opts);
  if (workspace_bytes < need || (need && !workspace)) return fail(FP4_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  hipStream_t s = (hipStream_t)stream;
  const int64_t B = prob->B, H = prob->H, Hkv = prob->Hkv, Sq = prob->Sq, Sk = prob->Sk, d = prob->d;
  MxAttnLaunch A;
  A.qc = prob->q_codes; A.qs = prob->q_scales; A.kc = prob->k_codes; A.ks = prob->k_scales;
  A.vc = prob->v_codes; A.vs = prob->v_scales;
  if (need) {
    char* ws = (char*)workspace;
    const size_t nq = (size_t)(B * H * Sq * d), nk = (size_t)(B * Hkv * Sk * d);
    uint8_t* qc = (uint8_t*)ws;
    uint8_t* qs = qc + align256(nq / 2);
    uint8_t* kc = qs + align256(nq / 32);
    uint8_t* ks = kc + align256(nk / 2);
    uint8_t* vc = ks + align256(nk / 32);
    uint8_t* vs = vc + align256(nk / 2);
    hipError_t e = fp4i_launch_mx_quantize(prob->q, prob->dtype, B * H * Sq, d, d, 0, qc, qs, s);
    if (e == hipSuccess) e = fp4i_launch_mx_quantize(prob->k, prob->dtype, B * Hkv * Sk, d, d, 0, kc, ks, s);
    // V blocks run along tokens; 32-token blocks never straddle heads (Sk % 32 == 0)
    if (e == hipSuccess) e = fp4i_launch_mx_quantize(prob->v, prob->dtype, B * Hkv * Sk, d, d, 1, vc, vs, s);
    if (e != hipSuccess) return hip_status(e, "fp4_attention_fwd_mx quantize launch");
    A.qc = qc; A.qs = qs; A.kc = kc; A.ks = ks; A.vc = vc; A.vs = vs;
  }
  A.B = B; A.H = H; A.Hkv = Hkv; A.Sq = Sq; A.Sk = Sk; A.d = d;
  A.causal = opts->causal;
  A.c = score_factor(opts->softmax_scale, d);
  A.kv_tile = opts->kv_tile;
  A.out_dtype = opts->out_dtype;
  A.out = out;
  A.lse = lse;
  return hip_status(fp4i_launch_attn_mx(A, s), "fp4_attention_fwd_mx launch");
}

size_t fp4_attention_bwd_workspace_size(const fp4_attn_problem* prob, const fp4_attn_opts* opts) {
  if (!prob || !opts || prob->struct_size < sizeof(fp4_attn_problem) || opts->struct_size < sizeof(fp4_attn_opts))
    return 0;
  const AttnPlan P = plan_attn(prob, opts);
  AttnBwdLaunch L{};
  L.B = prob->B; L.H = prob->H; L.Hkv = prob->Hkv; L.Sq = prob->Sq; L.Sk = prob->Sk; L.d = prob->d;
  return align256(P.total) + fp4i_attn_bwd_workspace(L);
}

int fp4_attention_bwd(const fp4_attn_problem* prob, const fp4_attn_opts* opts, const void* out_hp, const float* lse,
                      const void* dout, float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                      void* stream) {
  const char* fn = "fp4_attention_bwd";
  int st = check_attn(prob, opts, fn, false);
  if (st) return st;
  if (opts->fp16_budget_pct != 0) return fail(FP4_ERR_UNSUPPORTED, "%s: training has no FP16 path (fp16_budget_pct must be 0)", fn);
  if (opts->hadamard_qk) return fail(FP4_ERR_UNSUPPORTED, "%s: the rotation is not supported in training", fn);
  if (opts->balance_qk) return fail(FP4_ERR_UNSUPPORTED, "%s: the balance pair is not supported in training", fn);
  // the dK/dV kernels address one head's query rows through 32-bit buffer offsets
  if (prob->Sq * prob->d * 2 >= ((int64_t)1 << 31)) return fail(FP4_ERR_UNSUPPORTED, "%s: Sq * d too large", fn);
  if (!out_hp || !lse || !dout || !dq || !dk || !dv) return fail(FP4_ERR_INVALID_ARG, "%s: out_hp, lse, dout, dq, dk, dv are required", fn);
  const void* ptrs[] = {out_hp, lse, dout, dq, dk, dv};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return fail(FP4_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  const size_t need = fp4_attention_bwd_workspace_size(prob, opts);
  if (workspace_bytes < need || !workspace) return fail(FP4_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  const AttnPlan P = plan_attn(prob, opts);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int64_t B = prob->B, H = prob->H, Hkv = prob->Hkv, Sq = prob->Sq, Sk = prob->Sk, d = prob->d;
  const uint8_t *qc = prob->q_codes, *qs = prob->q_scales, *kc = prob->k_codes, *ks = prob->k_scales,
                *vc = prob->v_codes, *vs = prob->v_scales;
  if (P.need_quant) {  // the forward's quantization, repeated
    const Maps maps = maps_of(prob);
    QuantLaunch L{};
    L.dtype = prob->dtype;
    L.search = opts->scale_search;
    L.fmin = opts->f_min;
    L.fmax = opts->f_max;
    L.cols = d;
    L.ld = d;
    L.strided = maps.strided ? 1 : 0;
    L.map = maps.q;
    L.x = prob->q; L.rows = B * H * Sq; L.axis = 0;
    L.codes = (uint8_t*)(ws + P.qc); L.scales = (uint8_t*)(ws + P.qs);
    QuantLaunch LK = L;
    LK.x = prob->k; LK.rows = B * Hkv * Sk;
    LK.map = maps.k;
    LK.codes = (uint8_t*)(ws + P.kc); LK.scales = (uint8_t*)(ws + P.ks);
    QuantLaunch LV = LK;
    LV.x = prob->v; LV.axis = 1;
    LV.map = maps.v;
    LV.codes = (uint8_t*)(ws + P.vc); LV.scales = (uint8_t*)(ws + P.vs);
    const hipError_t e = fp4i_launch_quantize_qkv(L, LK, LV, s);
    if (e != hipSuccess) return hip_status(e, "fp4_attention_bwd quantize launch");
    qc = (uint8_t*)(ws + P.qc); qs = (uint8_t*)(ws + P.qs);
    kc = (uint8_t*)(ws + P.kc); ks = (uint8_t*)(ws + P.ks);
    vc = (uint8_t*)(ws + P.vc); vs = (uint8_t*)(ws + P.vs);
  }
  AttnBwdLaunch L{};
  L.B = B; L.H = H; L.Hkv = Hkv; L.Sq = Sq; L.Sk = Sk; L.d = d;
  L.dtype = prob->dtype;
  L.hp_dtype = opts->out_dtype;
  L.qc = qc; L.qs = qs; L.kc = kc; L.ks = ks; L.vc = vc; L.vs = vs;
  L.dout = dout;
  L.out_hp = out_hp;
  L.lse = lse;
  L.causal = opts->causal;
  L.kv_tile = opts->kv_tile;
  L.single = opts->p_single_level;
  L.c = score_factor(opts->softmax_scale, d);
  L.dq = dq; L.dk = dk; L.dv = dv;
  L.ws = ws + align256(P.total);
  return hip_status(fp4i_launch_attn_bwd(L, s), "fp4_attention_bwd launch");
}

int fp4_attention_fwd_train(const fp4_attn_problem* prob, const fp4_attn_opts* opts, void* out, void* out_hp,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "fp4_attention_fwd_train";
  int st = check_attn(prob, opts, fn, false);
  if (st) return st;
  if (opts->fp16_budget_pct != 0) return fail(FP4_ERR_UNSUPPORTED, "%s: training has no FP16 path (fp16_budget_pct must be 0)", fn);
  if (!out || !out_hp || !lse || !aligned16(out) || !aligned16(out_hp))
    return fail(FP4_ERR_INVALID_ARG, "%s: out, out_hp and lse are required (16-byte aligned)", fn);
  return attention_fwd_impl(prob, opts, out, out_hp, lse, nullptr, nullptr, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Workspace plan of a decode call: partials, then (with a budget) the
// selection's keys, indices, counts and block mask.
struct DecodePlan {
  int nsplit = 0, nfull = 0, nprom = 0, kmax = 0, nbc = 0, nbw = 0;
  int64_t split_len = 0;
  size_t part_o = 0, part_ml = 0, keys = 0, idx = 0, cnt = 0, mask = 0, total = 0;
};

DecodePlan decode_plan(int64_t Hq, const fp4_kv_cache* c, int pct) {
  DecodePlan P;
  P.nsplit = fp4i_decode_splits(c->B, c->Hkv, c->mid_cap, &P.split_len);
  P.nfull = fp4i_decode_full_splits((int64_t)c->n_sink + c->n_recent);
  if (pct > 0) {
    P.nbc = (int)((c->mid_cap + kDecSelBlock - 1) / kDecSelBlock);
    P.kmax = (pct * P.nbc + 99) / 100;
    P.nprom = (P.kmax + 3) / 4;
    P.nbw = (P.nbc + 31) / 32;
  }
  const size_t n = (size_t)(c->B * Hq) * (size_t)(P.nsplit + P.nfull + P.nprom);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align256(bytes); return at; };
  P.part_o = take(n * (size_t)c->d * sizeof(float));
  P.part_ml = take(n * 2 * sizeof(float));
  if (pct > 0) {
    const size_t nbk = (size_t)(c->B * c->Hkv);
    P.keys = take(nbk * (size_t)(P.nbc > 0 ? P.nbc : 1) * sizeof(uint64_t));
    P.idx = take(nbk * (size_t)(P.kmax > 0 ? P.kmax : 1) * sizeof(int32_t));
    P.cnt = take(nbk * sizeof(int32_t));
    P.mask = take(nbk * (size_t)(P.nbw > 0 ? P.nbw : 1) * sizeof(uint32_t));
  }
  P.total = off;
  return P;
}

bool decode_args_ok(int64_t Hq, const fp4_kv_cache* c) {
  return c && c->struct_size >= sizeof(fp4_kv_cache) && Hq > 0 && c->B > 0 && c->Hkv > 0 && c->d > 0 &&
         c->mid_cap >= 0;
}

int decode_impl(const char* fn, const void* q, int64_t Hq, const fp4_kv_cache* c, int pct, float softmax_scale,
                int32_t out_dtype, void* out, float* lse, int32_t* sel_idx, int32_t* sel_cnt, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (!c || c->struct_size < sizeof(fp4_kv_cache)) return fail(FP4_ERR_INVALID_ARG, "%s: cache is NULL or struct_size too small", fn);
  if (!q || !out) return fail(FP4_ERR_INVALID_ARG, "%s: q and out are required", fn);
  if (c->B < 1 || c->Hkv < 1 || Hq < 1 || Hq % c->Hkv) return fail(FP4_ERR_INVALID_ARG, "%s: bad B/Hq/Hkv", fn);
  if (c->d != 64 && c->d != 128) return fail(FP4_ERR_UNSUPPORTED, "%s: head dim %lld not in {64,128}", fn, (long long)c->d);
  if (Hq / c->Hkv > 16) return fail(FP4_ERR_UNSUPPORTED, "%s: more than 16 query heads per kv head", fn);
  if (c->n_sink < 0 || c->n_recent < 0 || c->mid_cap < 0 || c->mid_cap % 16)
    return fail(FP4_ERR_INVALID_ARG, "%s: n_sink/n_recent must be >= 0 and mid_cap a multiple of 16", fn);
  if (c->n_sink + c->n_recent + c->mid_cap < 1) return fail(FP4_ERR_INVALID_ARG, "%s: empty cache", fn);
  if (c->mid_cap * c->d / 2 >= ((int64_t)1 << 31)) return fail(FP4_ERR_UNSUPPORTED, "%s: mid_cap * d too large", fn);
  if ((c->n_sink && (!c->k_sink || !c->v_sink)) || (c->n_recent && (!c->k_recent || !c->v_recent)))
    return fail(FP4_ERR_INVALID_ARG, "%s: sink/recent buffers missing", fn);
  if (c->mid_cap && (!c->k_codes || !c->k_scales || !c->v_codes || !c->v_scales || !c->mid_len))
    return fail(FP4_ERR_INVALID_ARG, "%s: NVFP4 region buffers or mid_len missing", fn);
  if (out_dtype < FP4_BF16 || out_dtype > FP4_FP32) return fail(FP4_ERR_INVALID_ARG, "%s: bad out_dtype", fn);
  if (pct < 0 || pct > 100) return fail(FP4_ERR_INVALID_ARG, "%s: fp16_budget_pct must be in [0, 100]", fn);
  if (pct > 0 && c->mid_cap > 0 && (!c->k_mid || !c->v_mid || !c->k_sum))
    return fail(FP4_ERR_INVALID_ARG, "%s: a budget > 0 needs the full-precision copy (k_mid, v_mid, k_sum)", fn);
  const void* ptrs[] = {q, out, c->k_sink, c->v_sink, c->k_codes, c->k_scales, c->v_codes, c->v_scales, c->k_recent,
                        c->v_recent, pct > 0 ? c->k_mid : nullptr, pct > 0 ? c->v_mid : nullptr,
                        pct > 0 ? (const void*)c->k_sum : nullptr};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(FP4_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  const DecodePlan P = decode_plan(Hq, c, pct);
  if (workspace_bytes < P.total || !workspace) return fail(FP4_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, P.total);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  DecodeLaunch L{};
  L.q = q;
  L.B = c->B; L.Hq = Hq; L.Hkv = c->Hkv; L.d = c->d;
  L.n_sink = c->n_sink; L.n_recent = c->n_recent; L.mid_cap = c->mid_cap;
  L.k_sink = c->k_sink; L.v_sink = c->v_sink;
  L.kc = c->k_codes; L.ks = c->k_scales; L.vc = c->v_codes; L.vs = c->v_scales;
  L.k_recent = c->k_recent; L.v_recent = c->v_recent;
  L.mid_len = c->mid_len;
  L.c = score_factor(softmax_scale, c->d);
  L.out_dtype = out_dtype;
  L.out = out;
  L.lse = lse;
  L.nsplit = P.nsplit;
  L.split_len = P.split_len;
  L.nfull = P.nfull;
  L.part_o = (float*)(ws + P.part_o);
  L.part_ml = (float*)(ws + P.part_ml);
  if (pct > 0) {
    DecSelectLaunch S{};
    S.q = q;
    S.k_sum = c->k_sum;
    S.mid_len = c->mid_len;
    S.B = c->B; S.Hq = Hq; S.Hkv = c->Hkv; S.d = c->d; S.mid_cap = c->mid_cap;
    S.pct = pct; S.kmax = P.kmax; S.nbc = P.nbc; S.nbw = P.nbw;
    S.keys = (uint64_t*)(ws + P.keys);
    S.idx = sel_idx ? sel_idx : (int32_t*)(ws + P.idx);
    S.cnt = sel_cnt ? sel_cnt : (int32_t*)(ws + P.cnt);
    S.mask = (uint32_t*)(ws + P.mask);
    hipError_t e = fp4i_launch_decode_select(S, st);
    if (e != hipSuccess) return hip_status(e, "decode selection launch");
    L.k_mid = c->k_mid;
    L.v_mid = c->v_mid;
    L.sel_idx = S.idx;
    L.sel_mask = S.mask;
    L.kmax = P.kmax;
    L.nprom = P.nprom;
    L.nbw = P.nbw;
  }
  return hip_status(fp4i_launch_decode(L, st), "fp4_attention_decode launch");
}

}  // namespace

extern "C" {

size_t fp4_attention_decode_workspace_size(int64_t Hq, const fp4_kv_cache* c) {
  if (!decode_args_ok(Hq, c)) return 0;
  return decode_plan(Hq, c, 0).total;
}

int fp4_attention_decode(const void* q, int64_t Hq, const fp4_kv_cache* c, float softmax_scale,
                         int32_t out_dtype, void* out, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return decode_impl("fp4_attention_decode", q, Hq, c, 0, softmax_scale, out_dtype, out, lse, nullptr, nullptr,
                     workspace, workspace_bytes, stream);
}

size_t fp4_attention_decode_selective_workspace_size(int64_t Hq, const fp4_kv_cache* c, int32_t pct) {
  if (!decode_args_ok(Hq, c) || pct < 0 || pct > 100) return 0;
  return decode_plan(Hq, c, pct).total;
}

int fp4_attention_decode_selective(const void* q, int64_t Hq, const fp4_kv_cache* c, int32_t fp16_budget_pct,
                                   float softmax_scale, int32_t out_dtype, void* out, float* lse, int32_t* sel_idx,
                                   int32_t* sel_cnt, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl("fp4_attention_decode_selective", q, Hq, c, fp16_budget_pct, softmax_scale, out_dtype, out,
                     lse, sel_idx, sel_cnt, workspace, workspace_bytes, stream);
}

int fp4_kv_block_sums(const fp4_kv_cache* c, void* stream) {
  const char* fn = "fp4_kv_block_sums";
  if (!c || c->struct_size < sizeof(fp4_kv_cache)) return fail(FP4_ERR_INVALID_ARG, "%s: cache is NULL or struct_size too small", fn);
  if (c->B < 1 || c->Hkv < 1) return fail(FP4_ERR_INVALID_ARG, "%s: bad B/Hkv", fn);
  if (c->d != 64 && c->d != 128) return fail(FP4_ERR_UNSUPPORTED, "%s: head dim %lld not in {64,128}", fn, (long long)c->d);
  if (c->mid_cap < 0 || c->mid_cap % 16) return fail(FP4_ERR_INVALID_ARG, "%s: mid_cap must be a multiple of 16", fn);
  if (c->mid_cap == 0) return FP4_OK;
  if (!c->k_mid || !c->k_sum || !c->mid_len) return fail(FP4_ERR_INVALID_ARG, "%s: k_mid, k_sum and mid_len are required", fn);
  if (!aligned16(c->k_mid) || !aligned16(c->k_sum)) return fail(FP4_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  return hip_status(fp4i_launch_kv_block_sums(c->k_mid, c->mid_len, const_cast<double*>(c->k_sum), c->B, c->Hkv,
                                              c->mid_cap, c->d, (hipStream_t)stream),
                    "fp4_kv_block_sums launch");
}

size_t fp4_kv_cache_append_workspace_size(const fp4_kv_cache* c) {
  if (!c || c->struct_size < sizeof(fp4_kv_cache) || c->B <= 0 || c->Hkv <= 0 || c->d <= 0 || c->n_recent < 0)
    return 0;
  return fp4i_kv_append_workspace(c->B, c->Hkv, c->n_recent, c->d);
}

int fp4_kv_cache_append(const fp4_kv_cache* c, const void* k_new, const void* v_new, int32_t n_new,
                        int32_t* overflow, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "fp4_kv_cache_append";
  if (!c || c->struct_size < sizeof(fp4_kv_cache)) return fail(FP4_ERR_INVALID_ARG, "%s: cache is NULL or struct_size too small", fn);
  if (c->B < 1 || c->Hkv < 1) return fail(FP4_ERR_INVALID_ARG, "%s: bad B/Hkv", fn);
  if (c->d != 64 && c->d != 128) return fail(FP4_ERR_UNSUPPORTED, "%s: head dim %lld not in {64,128}", fn, (long long)c->d);
  if (n_new <= 0 || n_new % 16) return fail(FP4_ERR_INVALID_ARG, "%s: n_new must be a positive multiple of 16", fn);
  if (c->n_recent < 0 || c->mid_cap < 16 || c->mid_cap % 16)
    return fail(FP4_ERR_INVALID_ARG, "%s: need n_recent >= 0 and a NVFP4 capacity that is a positive multiple of 16", fn);
  if (c->mid_cap * c->d / 2 >= ((int64_t)1 << 31)) return fail(FP4_ERR_UNSUPPORTED, "%s: mid_cap * d too large", fn);
  if (!k_new || !v_new) return fail(FP4_ERR_INVALID_ARG, "%s: k_new and v_new are required", fn);
  if (c->n_recent && (!c->k_recent || !c->v_recent)) return fail(FP4_ERR_INVALID_ARG, "%s: recent buffers missing", fn);
  if (!c->k_codes || !c->k_scales || !c->v_codes || !c->v_scales || !c->mid_len)
    return fail(FP4_ERR_INVALID_ARG, "%s: NVFP4 region buffers or mid_len missing", fn);
  const int ndual = (c->k_mid ? 1 : 0) + (c->v_mid ? 1 : 0) + (c->k_sum ? 1 : 0);
  if (ndual != 0 && ndual != 3) return fail(FP4_ERR_INVALID_ARG, "%s: give all of k_mid, v_mid, k_sum or none", fn);
  const void* ptrs[] = {k_new, v_new, c->k_recent, c->v_recent, c->k_codes, c->k_scales, c->v_codes, c->v_scales,
                        c->k_mid, c->v_mid, c->k_sum};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(FP4_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  const size_t need = fp4_kv_cache_append_workspace_size(c);
  if (workspace_bytes < need || !workspace) return fail(FP4_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  KvAppendLaunch L;
  L.B = c->B; L.Hkv = c->Hkv; L.d = c->d; L.mid_cap = c->mid_cap;
  L.n_recent = c->n_recent; L.n_new = n_new;
  L.k_new = k_new; L.v_new = v_new;
  L.k_recent = const_cast<void*>(c->k_recent);
  L.v_recent = const_cast<void*>(c->v_recent);
  L.kc = const_cast<uint8_t*>(c->k_codes); L.ks = const_cast<uint8_t*>(c->k_scales);
  L.vc = const_cast<uint8_t*>(c->v_codes); L.vs = const_cast<uint8_t*>(c->v_scales);
  L.mid_len = const_cast<int32_t*>(c->mid_len);
  L.overflow = overflow;
  L.ws = workspace;
  L.k_mid = const_cast<void*>(c->k_mid);
  L.v_mid = const_cast<void*>(c->v_mid);
  L.k_sum = const_cast<double*>(c->k_sum);
  return hip_status(fp4i_launch_kv_append(L, (hipStream_t)stream), "fp4_kv_cache_append launch");
}

}  // extern "C"

/*
 * fp4.h -- C ABI of the block-scaled FP4 attention library for AMD MI355X (gfx950).
 *
 * The library quantizes tensors to NVFP4-style blocks (4-bit E2M1 elements,
 * one E4M3 scale per 16 elements, optional per-tensor binary32 scale), runs a
 * fused flash-style attention forward on those operands with two-level
 * quantization of the probabilities and an FP16 path for selected block pairs,
 * and decodes one token against a KV cache that keeps its first and last
 * tokens in bf16 and the rest in NVFP4.
 *
 * Sources (web pages, cited by title and section):
 *   ScaleSearch page  -- "Busca tus escalas de punto flotante por bloques":
 *     Declaracion del Problema (NVFP4 format), Metodologia / ScaleSearch
 *     (max-scaling and the offset search), Metodologia / ScaleSearchAttention
 *     (NVFP4 QK^T and PV with FP32 accumulation; sink-aware cache precision).
 *   ThriftAttention page -- Metodologia / 1 (block means, mean-dot-product
 *     scores, top-k block pairs) and / 2 (FP16 path for the selected pairs, FP4
 *     path with two-level P for the others, fused by an online softmax).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are device pointers owned by the caller; option structs
 *     are host pointers.  The library never allocates, frees or retains caller
 *     memory.  Scratch memory comes from a caller workspace whose size the
 *     matching *_workspace_size() query returns (0 means none is needed).
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream) and the call returns without synchronizing.
 *   - Arguments are validated before anything is launched.  On error nothing
 *     runs and a negative status is returned; fp4_last_error() then returns a
 *     message for the calling thread.  No exception or abort crosses the ABI.
 *   - Calls that share a workspace buffer must be ordered on one stream.
 *   - Every option struct starts with struct_size = sizeof(struct), so that
 *     the struct can grow without breaking callers.
 *   - Debug switches, read from the environment at every call: FP4_LOG=1
 *     prints each launch and each error on stderr; FP4_SYNC_CHECK=1 waits for
 *     the device after each launch (hipDeviceSynchronize), so an error raised
 *     while a kernel runs is returned as FP4_ERR_HIP by the call that launched
 *     it instead of surfacing at a later call.
 */
#ifndef FP4_H
#define FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define FP4_OK 0
#define FP4_ERR_INVALID_ARG (-1) /* null pointer, bad shape, bad option */
#define FP4_ERR_UNSUPPORTED (-2) /* valid request the kernels do not cover (e.g. head dim) */
#define FP4_ERR_WORKSPACE (-3)   /* workspace missing or smaller than the query returned */
#define FP4_ERR_HIP (-4)         /* a HIP runtime call failed */

/* element types of high-precision tensors */
#define FP4_BF16 0
#define FP4_FP16 1
#define FP4_FP32 2

/* per-tensor (second-level) scale modes of fp4_quantize */
#define FP4_GLOBAL_NONE 0  /* g = 1 */
#define FP4_GLOBAL_AMAX 1  /* g = amax(|x|) / 2688 computed on the device (2688 = 6 * 448) */
#define FP4_GLOBAL_GIVEN 2 /* g read from *g; elements are multiplied by 1/g first */

/* Library version, major * 10000 + minor * 100 + patch. */
int fp4_version(void);

/* Message describing the last failed call on this thread ("" if none). */
const char* fp4_last_error(void);

/* ------------------------------------------------------------------------ */
/* Quantization -- ScaleSearch page, Metodologia / ScaleSearch               */
/* ------------------------------------------------------------------------ */

typedef struct fp4_quant_opts {
  uint32_t struct_size; /* sizeof(fp4_quant_opts) */
  int32_t scale_search; /* 0: max-scaling only; 1: offset search */
  int32_t f_min;        /* offset search range, -8 <= f_min <= 0 <= f_max <= 8 (default -2, 6) */
  int32_t f_max;
  int32_t global_scale; /* FP4_GLOBAL_* */
  int32_t block_axis;   /* 0: blocks of 16 consecutive columns; 1: of 16 consecutive rows */
  /* Incoherence processing (ScaleSearch page, Metodologia / ScaleSearchAttention:
     Hadamard transforms before quantization, as in QuIP#).  1: every row
     is first replaced by H_n (s o row) / sqrt(n), n = cols, s_j = -1 where bit
     j of hadamard_signs is set (bit j % 32 of word j / 32), H_n the Sylvester
     Hadamard matrix applied by binary32 butterfly stages of span 1, 2, 4, ...
     (pair (i, i+h) -> (a + b, a - b)), then a multiply by the binary32 value
     of 1/sqrt(n).  Needs block_axis 0, cols in {16, 32, 64, 128} and a global
     scale mode other than FP4_GLOBAL_AMAX.  0: off. */
  int32_t hadamard;
  uint32_t hadamard_signs[4];
  /* Magnitude balance (ScaleSearch page, Metodologia / ScaleSearchAttention:
     a pair Q' = Q R^-T, K' = K R that keeps Q K^T, here with R = diag(2^e)).
     NULL: off.  Otherwise a device array of int32 exponents
     [rows / exp_rows][cols] (e.g. from fp4_qk_balance): every element of row
     r is first multiplied by 2^(e[r / exp_rows][col]), by 2^-e when exp_negate
     is 1 (the Q side), exactly in binary32, before the rotation and the
     per-tensor factor.  Needs block_axis 0, exp_rows >= 1 dividing rows, and a
     global scale mode other than FP4_GLOBAL_AMAX. */
  const int32_t* channel_exp;
  int32_t exp_negate;
  int64_t exp_rows;
} fp4_quant_opts;

/*
 * Quantize x [rows, cols] (row stride ld >= cols elements, dtype FP4_BF16,
 * FP4_FP16 or FP4_FP32) into 16-element blocks.
 *
 * Per block: a = max|y| with y = x (or x * 1/g); scale s0 = a/6 rounded to the
 * nearest E4M3 value (ties to even, saturating at 448).  With scale_search,
 * candidate scale bytes s0 + f for f in [f_min, f_max] (bytes outside 0..0x7E
 * skipped) are tried and the one with the least squared error is kept, the
 * lowest f on ties.  Elements are |y| times the correctly rounded reciprocal
 * of the scale, rounded to the nearest E2M1 value (ties to even); the sign bit
 * of y is kept.  A block holding Inf/NaN gets scale byte 0x7F and zero codes.
 *
 * Outputs (dense, device):
 *   block_axis 0: codes [rows, cols/2] (element 2i in the low nibble),
 *                 scales and offsets [rows, cols/16]
 *   block_axis 1: codes [rows/2, cols] (row 2i in the low nibble),
 *                 scales and offsets [rows/16, cols]
 *   offsets (nullable) receive the chosen f as int8.
 *   g: FP4_GLOBAL_NONE -- nullable, set to 1.0 when given;
 *      FP4_GLOBAL_AMAX -- required, receives amax/2688 (1.0 for an all-zero
 *        tensor; NaN elements are ignored by the maximum);
 *      FP4_GLOBAL_GIVEN -- required, read (must be finite and > 0).
 * Requirements: cols % 16 == 0 for block_axis 0, rows % 16 == 0 for
 * block_axis 1; x, codes, scales 16-byte aligned.  Workspace: see
 * fp4_quantize_workspace_size (non-zero only for FP4_GLOBAL_AMAX).
 * Dequantized value: E2M1(code) * E4M3(scale) * g.
 */
int fp4_quantize(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                 const fp4_quant_opts* opts, uint8_t* codes, uint8_t* scales, int8_t* offsets,
                 float* g, void* workspace, size_t workspace_bytes, void* stream);

size_t fp4_quantize_workspace_size(int64_t rows, int64_t cols, const fp4_quant_opts* opts);

/*
 * MXFP4 variant: E2M1 elements with one power-of-two scale per 32 elements
 * (the block floating point the ScaleSearch page contrasts NVFP4 with,
 * Declaracion del Problema; the operand format of gfx950's FP4 matrix
 * instructions).  Scale byte = E8M0 (value 2^(byte - 127)) with the OCP
 * microscaling rule: exponent floor(log2(amax)) - 2 clamped to [-127, 127]
 * (byte 0 for an all-zero block, 0xFF for a block holding Inf/NaN, whose
 * codes are then 0); elements |x| / 2^exponent rounded to the nearest E2M1
 * value (ties to the even code, saturating at 6), sign bit copied.
 * Layouts as fp4_quantize with blocks of 32: block_axis 0 -> codes
 * [rows, cols/2], scales [rows, cols/32]; block_axis 1 -> codes
 * [rows/2, cols], scales [rows/32, cols].  No offset search, no per-tensor
 * scale, no workspace.
 */
int fp4_mx_quantize(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld, int32_t block_axis,
                    uint8_t* codes, uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------ */
/* Attention forward -- ScaleSearch page, Metodologia / ScaleSearchAttention; */
/* ThriftAttention page, Metodologia / 1 and 2                               */
/* ------------------------------------------------------------------------ */

typedef struct fp4_attn_problem {
  uint32_t struct_size; /* sizeof(fp4_attn_problem) */
  int64_t B, H, Hkv;    /* batch, query heads, key/value heads (H % Hkv == 0) */
  int64_t Sq, Sk, d;    /* query / key lengths, head dimension (64 or 128) */
  int32_t dtype;        /* FP4_BF16 or FP4_FP16 for q, k, v */
  /* high-precision inputs: q [B,H,Sq,d], k and v [B,Hkv,Sk,d], dense unless
     their strides below are given.  Needed unless all six quantized arrays
     below are given; always needed when fp16_budget_pct > 0 (block means and
     the FP16 path read them). */
  const void* q;
  const void* k;
  const void* v;
  /* optional NVFP4 operands from fp4_quantize (all six or none), dense:
     q: codes [B,H,Sq,d/2], scales [B,H,Sq,d/16]      (blocks along d)
     k: codes [B,Hkv,Sk,d/2], scales [B,Hkv,Sk,d/16]  (blocks along d)
     v: codes [B,Hkv,Sk/2,d], scales [B,Hkv,Sk/16,d]  (blocks of 16 tokens)
     When absent they are produced in the workspace with the opts' search. */
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  /* Element strides {batch, head, token} of q, k and v; all three zero means
     dense.  A token's d elements stay contiguous.  Strides must be >= 0, the
     token stride >= d, all multiples of 8 elements (whole 16-byte rows), and
     for k and v ((S - 1) * token stride + d) * 2 < 2^31.  Example, a fused
     projection [B, S, H + 2 Hkv, d]: q = base, k = base + H d,
     v = base + (H + Hkv) d, each with strides {S (H + 2 Hkv) d, d,
     (H + 2 Hkv) d}.  Read by the call's own quantization, the block means,
     the balance exponents and the FP16 path, in the same launches as dense
     inputs (no copy); fp4_attention_fwd_mx needs dense inputs. */
  int64_t q_strides[3];
  int64_t k_strides[3];
  int64_t v_strides[3];
} fp4_attn_problem;

typedef struct fp4_attn_opts {
  uint32_t struct_size;    /* sizeof(fp4_attn_opts) */
  int32_t causal;          /* 1: key j visible to query i iff j <= i (needs Sq == Sk) */
  float softmax_scale;     /* <= 0 selects 1/sqrt(d) */
  int32_t kv_tile;         /* 64 or 128 keys: the group of the row-level P scale */
  int32_t scale_search;    /* quantization of q, k, v done inside the call */
  int32_t f_min, f_max;
  int32_t fp16_budget_pct; /* 0..100: share of visible key blocks per query block on the FP16 path */
  int32_t sel_block;       /* selection block (tokens), 128; multiple of kv_tile */
  int32_t out_dtype;       /* FP4_BF16, FP4_FP16 or FP4_FP32 */
  int32_t selection_given; /* 1: topk_idx/topk_cnt are inputs (e.g. from fp4_block_topk) and
                              no selection is computed; 0: the call computes the selection */
  int32_t hadamard_qk;     /* 1: the call quantizes Q and K after the rotation of fp4_quant_opts'
                              hadamard (n = d) with these signs; QK^T is kept, the FP16 path
                              and the block means use the original Q and K.  Needs the call
                              to quantize (no pre-quantized operands). */
  uint32_t hadamard_signs[4];
  int32_t p_single_level;  /* 1: the FP4 path quantizes P with the NVFP4 block scale alone,
                              s2 = E4M3(amax(e) / 6) per 16 keys and codes RNE_E2M1(e / s2)
                              (Attn-QAT page, Metodologia / B: no two-level step); 0: the
                              two-level P above */
  int32_t balance_qk;      /* 1: the call quantizes Q' = Q 2^-e and K' = K 2^e with the
                              exponents of fp4_qk_balance (before the rotation when hadamard_qk
                              is on); QK^T is kept exactly, the FP16 path and the block means use
                              the original Q and K.  Needs the call to quantize. */
} fp4_attn_opts;

/*
 * out [B,H,Sq,d] = softmax(scale * q k^T) v with fake-quant NVFP4 numerics:
 * per (query row, key tile) of kv_tile keys, x = fl32(S * log2(e) * scale),
 * e = 2^(x - tile row max); on the FP4 path the row level maps e = 1 to 2688
 * and each 16-key block of P takes an E4M3 scale s2 = E4M3(amax(e) * 448)
 * with elements e * (2688/s2) rounded to E2M1; the tile adds P^ V^ / 2688.
 * On the FP16 path (selected pairs) the tile adds fp16(e) fp16(v) using
 * fp16(q) fp16(k) scores.  Tiles merge with an online softmax whose
 * denominator sums the unquantized e.  lse [B,H,Sq] (nullable) receives the
 * natural-log sum of exp of the scaled scores.
 * Selection (fp16_budget_pct > 0): per query block i of sel_block rows, the
 * visible key blocks j are scored by mean(q_i) . mean(k_j) in binary64 (one
 * fused multiply-add per channel, ascending channels) and the
 * ceil(pct * n_i / 100) best are kept (ties: lower j).  topk_idx
 * [B,H,ceil(Sq/sel_block),kmax] (ascending, -1 padded, kmax =
 * ceil(pct * ceil(Sk/sel_block) / 100)) and topk_cnt [B,H,ceil(Sq/sel_block)]
 * are written when non-null (otherwise kept in the workspace); with
 * opts->selection_given they are read instead and must both be non-null.
 * A given selection should list, per query block, distinct visible key-block
 * indices in ascending order with topk_cnt <= kmax.  What the kernel does with
 * any other list: topk_cnt is clamped to [0, kmax]; of the first topk_cnt
 * entries, only those greater than every entry before them are promoted
 * (negative, repeated and out-of-order entries are ignored), and indices at or
 * past ceil(Sk/sel_block) are ignored.  So no key is ever counted twice.
 * Requirements: d in {64, 128}; Sk % 16 == 0; causal needs Sq == Sk;
 * sel_block % kv_tile == 0; 16-byte aligned tensors.
 */
int fp4_attention_fwd(const fp4_attn_problem* prob, const fp4_attn_opts* opts, void* out,
                      float* lse, int32_t* topk_idx, int32_t* topk_cnt, void* workspace,
                      size_t workspace_bytes, void* stream);

size_t fp4_attention_fwd_workspace_size(const fp4_attn_problem* prob, const fp4_attn_opts* opts);

/* Block selection alone (the first stage of fp4_attention_fwd); needs prob->q
   and prob->k and fp16_budget_pct > 0.  Outputs as for fp4_attention_fwd. */
int fp4_block_topk(const fp4_attn_problem* prob, const fp4_attn_opts* opts, int32_t* topk_idx,
                   int32_t* topk_cnt, void* workspace, size_t workspace_bytes, void* stream);

size_t fp4_block_topk_workspace_size(const fp4_attn_problem* prob, const fp4_attn_opts* opts);

/*
 * Exponents of the magnitude-balancing pair Q' = Q R^-T, K' = K R (ScaleSearch
 * page, Metodologia / ScaleSearchAttention: a pair of linear maps that keeps
 * the attention scores and lowers the mean squared magnitude of Q and K).
 * R = diag(2^e) per (batch, kv head): ms_q[c] is the mean of q^2 over the
 * group's Hq/Hkv query heads and all Sq tokens, ms_k[c] the mean of k^2 over
 * the kv head's Sk tokens (binary64 sums), and e_c is the integer in [-8, 8]
 * minimizing ms_q 4^-e + ms_k 4^e: the smallest e with 4^(2e+1) >= ms_q/ms_k
 * (0 when either mean square is 0).  Because the entries are powers of two,
 * Q' and K' are exact in binary32 and Q' K'^T = Q K^T.
 * exponents: device int32 [B, Hkv, d] (written).  Needs prob->q and prob->k
 * (bf16 or fp16, dense).  The binary64 sums are reduced in a parallel order;
 * an exponent can depend on that order only when ms_q/ms_k lies within a few
 * units in the last place of a boundary 4^(2e+1).
 */
int fp4_qk_balance(const fp4_attn_problem* prob, int32_t* exponents, void* workspace, size_t workspace_bytes,
                   void* stream);

size_t fp4_qk_balance_workspace_size(const fp4_attn_problem* prob);

/*
 * MXFP4 variant of the forward (blocks of 32 with power-of-two scales, the
 * format the ScaleSearch page contrasts NVFP4 with, Declaracion del Problema;
 * gfx950's FP4 matrix instructions take its scales natively).  Q and K are
 * quantized with fp4_mx_quantize along d, V along tokens; per (query row, key
 * tile) x = fl32(S * log2(e) * scale), the tile reference is ceil(max x) (a
 * power of two that the E8M0 block scales can carry), e = 2^(x - ceil(max
 * x)), and each 32-key block of e is quantized by the rule of
 * fp4_mx_quantize; the tile adds P^ V^, tiles merge by online softmax over
 * the unquantized e.  Uses prob (q, k, v, or all six operands from
 * fp4_mx_quantize: q codes [B,H,Sq,d/2] scales [B,H,Sq,d/32], k codes
 * [B,Hkv,Sk,d/2] scales [B,Hkv,Sk,d/32], v codes [B,Hkv,Sk/2,d] scales
 * [B,Hkv,Sk/32,d]) and opts' causal, softmax_scale, kv_tile and out_dtype;
 * fp16_budget_pct and hadamard_qk must be 0, p_single_level and the scale
 * search fields are ignored.  Requirements as fp4_attention_fwd with
 * Sk % 32 == 0.  out, lse as fp4_attention_fwd.
 */
int fp4_attention_fwd_mx(const fp4_attn_problem* prob, const fp4_attn_opts* opts, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

size_t fp4_attention_fwd_mx_workspace_size(const fp4_attn_problem* prob, const fp4_attn_opts* opts);

/* ------------------------------------------------------------------------ */
/* Training -- Attn-QAT page, Metodologia / A (principles: P recomputed in    */
/* FP4 in the backward; a high-precision output O' for the softmax gradient) */
/* and / B (fake-quantized forward)                                          */
/* ------------------------------------------------------------------------ */

/*
 * Training forward: out and lse exactly as fp4_attention_fwd, and out_hp
 * [B,H,Sq,d] (opts->out_dtype) the high-precision output O' = P V^: the same
 * scores and softmax, with the probabilities themselves (as fp16 operands of
 * the product, not their FP4 version) weighting the fake-quantized V.  Needs
 * fp16_budget_pct == 0.  lse is required.  Workspace: fp4_attention_fwd's.
 */
int fp4_attention_fwd_train(const fp4_attn_problem* prob, const fp4_attn_opts* opts, void* out, void* out_hp,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training backward with straight-through fake quantization: given dout
 * [B,H,Sq,d] (prob->dtype), out_hp and lse from fp4_attention_fwd_train with
 * the same problem and opts, writes the binary32 gradients
 *   dv [B,Hkv,Sk,d] = P^T dO        (P^ the FP4 weights the forward used,
 *                                     recomputed in FP4)
 *   dq [B,H,Sq,d]   = dS K^,  dk [B,Hkv,Sk,d] = dS^T Q^ (summed over the
 *                    query heads of each kv head),
 *   dS = c ln2 * P * (dO V^T - rowsum(dO * O')),  P = 2^(x - lse log2 e),
 * with Q^, K^, V^ the NVFP4 operands of the forward (quantized again here
 * unless given).  Needs fp16_budget_pct == 0 and no rotation.  The scores
 * are recomputed, never stored: the workspace holds bfloat16 copies of Q^,
 * K^ and V^ (exact, as every E2M1 x E4M3 product has at most six significant
 * bits), dO as one bfloat16 term or, for binary16 dO, as two bfloat16 terms
 * whose sum is exact, and one float per query row (see the query).
 * FP4_ERR_UNSUPPORTED when Sq * d * 2 >= 2^31 (one head's query rows are
 * addressed through 32-bit byte offsets), as for Sk * d.
 */
int fp4_attention_bwd(const fp4_attn_problem* prob, const fp4_attn_opts* opts, const void* out_hp, const float* lse,
                      const void* dout, float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                      void* stream);

size_t fp4_attention_bwd_workspace_size(const fp4_attn_problem* prob, const fp4_attn_opts* opts);

/* ------------------------------------------------------------------------ */
/* Decode -- ScaleSearch page, Metodologia / ScaleSearchAttention (cache)    */
/* ------------------------------------------------------------------------ */

typedef struct fp4_kv_cache {
  uint32_t struct_size; /* sizeof(fp4_kv_cache) */
  int64_t B, Hkv, d;    /* batch, key/value heads, head dim (64 or 128) */
  int32_t n_sink;       /* bf16 tokens at the start of every context */
  int32_t n_recent;     /* bf16 tokens at the end of every context */
  int64_t mid_cap;      /* NVFP4 capacity in tokens (multiple of 16) */
  const void* k_sink;   /* bf16 [B,Hkv,n_sink,d] */
  const void* v_sink;
  const uint8_t* k_codes;  /* [B,Hkv,mid_cap,d/2]  blocks along d */
  const uint8_t* k_scales; /* [B,Hkv,mid_cap,d/16] */
  const uint8_t* v_codes;  /* [B,Hkv,mid_cap/2,d]  blocks of 16 tokens */
  const uint8_t* v_scales; /* [B,Hkv,mid_cap/16,d] */
  const void* k_recent;    /* bf16 [B,Hkv,n_recent,d], oldest first */
  const void* v_recent;
  const int32_t* mid_len;  /* device [B]: NVFP4 tokens in use, multiple of 16, <= mid_cap;
                              the context of batch b is n_sink + mid_len[b] + n_recent tokens */
  /* Optional full-precision copy of the middle (the dual cache of the
     ThriftAttention page, Significado: an FP16 and an FP4 copy side by side):
     all three pointers or none.  Read by fp4_attention_decode_selective with a
     budget > 0; fp4_kv_cache_append keeps them up to date when present. */
  const void* k_mid;       /* bf16 [B,Hkv,mid_cap,d]: the middle tokens unquantized */
  const void* v_mid;       /* bf16 [B,Hkv,mid_cap,d] */
  const double* k_sum;     /* [B,Hkv,ceil(mid_cap/128),d]: binary64 sum of each block of
                              FP4_DECODE_SEL_BLOCK k_mid tokens counted from the first middle
                              token (the last block in use may be short), added in ascending
                              token order */
} fp4_kv_cache;

/* tokens per selection block of the cache middle */
#define FP4_DECODE_SEL_BLOCK 128

/*
 * One query token per (batch, query head) against the cache: out [B,Hq,d] =
 * softmax(scale * q K^T) V over sink (bf16), middle (dequantized NVFP4) and
 * recent (bf16) tokens; query head h reads key/value head h / (Hq / Hkv).
 * q is bf16 [B,Hq,d] and is not quantized.  lse [B,Hq] is nullable.
 * mid_len values outside [0, mid_cap] are clamped and rounded down to a
 * multiple of 16 (no out-of-range reads).  Workspace: see the query.
 */
int fp4_attention_decode(const void* q, int64_t Hq, const fp4_kv_cache* cache, float softmax_scale,
                         int32_t out_dtype, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream);

size_t fp4_attention_decode_workspace_size(int64_t Hq, const fp4_kv_cache* cache);

/* Bytes of the fixed device array behind fp4_attention_decode_noalloc (one
   copy per GPU, held until the process ends). */
#define FP4_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * fp4_attention_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, kernels and results, with the workspace
 * taken from a fixed device array of the library (FP4_NOALLOC_SCRATCH_BYTES
 * per GPU) instead of a caller buffer.  The caller still owns q, the cache,
 * out and lse.  Calls no allocating routine.  A problem whose workspace
 * (fp4_attention_decode_workspace_size) exceeds the array is rejected with
 * FP4_ERR_UNSUPPORTED before anything runs.  All calls on one GPU share its
 * array: calls that overlap on a GPU (other streams, other threads) race and
 * must be serialized by the caller.
 */
int fp4_attention_decode_noalloc(const void* q, int64_t Hq, const fp4_kv_cache* cache, float softmax_scale,
                                 int32_t out_dtype, void* out, float* lse, void* stream);

/*
 * Decode with selective promotion (ThriftAttention page, Metodologia / 1 and
 * / 2, applied to one query token).  For every (batch, kv head) the middle is
 * cut into blocks of FP4_DECODE_SEL_BLOCK tokens from its first token (the
 * last one may be short: n_b = ceil(mid_len[b] / 128) blocks).  Block j is
 * scored by qbar . (k_sum[j] / tokens in j) in binary64, one fused multiply-add
 * per channel in ascending order,
 * where qbar is the mean of the kv head's G query vectors (reading: the query
 * block of a kv head is the G query tokens that read it).  The
 * ceil(fp16_budget_pct * n_b / 100) best blocks (ties: lower j) are read from
 * k_mid / v_mid, every other middle block from the NVFP4 copy; sink and recent
 * tokens as in fp4_attention_decode, and probabilities as there.
 * fp16_budget_pct 0..100; 0 is fp4_attention_decode (the dual pointers are
 * then not read).  sel_idx [B,Hkv,kmax] (ascending, -1 padded; kmax =
 * ceil(pct * ceil(mid_cap/128) / 100)) and sel_cnt [B,Hkv] receive the choice
 * when non-null.  k_sum must hold the sums of the tokens in use (see
 * fp4_kv_block_sums); NaN sums give an unspecified choice.  Workspace: see
 * the query (it depends on the budget).
 */
int fp4_attention_decode_selective(const void* q, int64_t Hq, const fp4_kv_cache* cache, int32_t fp16_budget_pct,
                                   float softmax_scale, int32_t out_dtype, void* out, float* lse, int32_t* sel_idx,
                                   int32_t* sel_cnt, void* workspace, size_t workspace_bytes, void* stream);

size_t fp4_attention_decode_selective_workspace_size(int64_t Hq, const fp4_kv_cache* cache,
                                                     int32_t fp16_budget_pct);

/*
 * (Re)computes cache->k_sum from cache->k_mid: for every (batch, kv head) and
 * block j < ceil(mid_cap/128), the binary64 sum over ascending tokens of the
 * block's tokens below mid_len[b] (0.0 for a block with none).  For a cache
 * whose middle was filled without fp4_kv_cache_append.  k_sum is written in
 * place.  No workspace.
 */
int fp4_kv_block_sums(const fp4_kv_cache* cache, void* stream);

/* ------------------------------------------------------------------------ */
/* Cache append -- ScaleSearch page, Metodologia / ScaleSearchAttention      */
/* (the middle of the cache is NVFP4 with ScaleSearch, its first and last   */
/* blocks full precision)                                                     */
/* ------------------------------------------------------------------------ */

/*
 * Quantize-on-write: appends n_new tokens (a multiple of 16) per (batch, kv
 * head).  For every batch b the recent window followed by the new tokens is a
 * sequence T of n_recent + n_new tokens; its first n_new tokens move into the
 * NVFP4 region at token mid_len[b] (K quantized per token in blocks of 16
 * channels, V in blocks of 16 tokens per channel, both with ScaleSearch over
 * offsets [-2, 6] and no per-tensor scale, exactly as fp4_quantize), the
 * recent window becomes the last n_recent tokens of T (oldest first), and
 * mid_len[b] becomes mid_len[b] + n_new (mid_len is first clamped to
 * [0, mid_cap] and rounded down to a multiple of 16, as the decode reads it).
 * A batch whose NVFP4 region has no room for n_new more tokens is left
 * unchanged; overflow [B] (device, nullable) receives 1 for such a batch, 0
 * otherwise.  The sink is never touched.  With the cache's full-precision
 * copy, the moved tokens are also written unquantized to k_mid / v_mid and
 * added, in token order, to the k_sum of their block (a block's sum restarts
 * from zero at its first token).
 * k_new, v_new: bf16 [B,Hkv,n_new,d], dense, 16-byte aligned.  The cache's
 * recent buffers, NVFP4 arrays and mid_len are written in place (the const
 * qualifiers of fp4_kv_cache do not apply to this call).  Calls on one cache
 * must be ordered on one stream.  Workspace: see the query (a copy of the
 * windows and one int per batch).
 */
int fp4_kv_cache_append(const fp4_kv_cache* cache, const void* k_new, const void* v_new, int32_t n_new,
                        int32_t* overflow, void* workspace, size_t workspace_bytes, void* stream);

size_t fp4_kv_cache_append_workspace_size(const fp4_kv_cache* cache);

#ifdef __cplusplus
}
#endif

#endif /* FP4_H */

// fp4_internal.h -- launch descriptors shared by the host API and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Element offsets of the token rows of a [B, Hn, S, d] tensor with strides
// (token ts, head hs, batch bs; the d elements of a row are contiguous).
// Dense: ts = d, hs = S d, bs = Hn S d.
struct TokMap {
  int64_t ts = 0, hs = 0, bs = 0;
  int64_t S = 1, Hn = 1;
  __host__ __device__ int64_t head_off(int64_t bh) const { return (bh / Hn) * bs + (bh % Hn) * hs; }
  __host__ __device__ int64_t row_off(int64_t r) const {
    const int64_t bh = r / S;
    return head_off(bh) + (r - bh * S) * ts;
  }
};

inline TokMap dense_map(int64_t Hn, int64_t S, int64_t d) {
  TokMap m;
  m.ts = d;
  m.hs = S * d;
  m.bs = Hn * S * d;
  m.S = S;
  m.Hn = Hn;
  return m;
}

struct QuantLaunch {
  const void* x;
  int dtype;  // 0 bf16, 1 fp16, 2 fp32
  int64_t rows, cols, ld;
  int axis;
  int search, fmin, fmax, gmode;
  uint8_t* codes;
  uint8_t* scales;
  int8_t* offsets;
  float* g;
  float* amax_ws;  // fp4i_amax_parts floats (mode 1)
  int hadamard;            // rotate rows (axis 0) before quantizing
  uint32_t hsigns[4];      // sign bits of the rotation
  float hscale;            // binary32 1/sqrt(cols)
  const int32_t* cexp;     // balance exponents [rows / exp_rows][cols], or null (axis 0)
  int exp_negate;          // 1: multiply by 2^-e (Q side)
  int64_t exp_rows;        // rows sharing one exponent vector
  // block means of the input, written in the same launch (axis 0, bf16/fp16,
  // cols <= 128, gmode 0): rows are heads of mS rows cut into mnb blocks of
  // mblk; means [rows / mS][mnb][cols] in binary64.  Null: none.
  double* means = nullptr;
  int64_t mS = 0;
  int mblk = 0, mnb = 0;
  // strided rows (attention inputs): row r at map.row_off(r) instead of r * ld
  int strided = 0;
  TokMap map;
};

// Balance exponents: per (batch, kv head) binary64 partial sums of squares of
// Q (the group's heads) and K over chunks of rows, then the exponents.
struct BalanceLaunch {
  const void* q;  // [B, H, Sq, d]
  const void* k;  // [B, Hkv, Sk, d]
  int dtype;      // 0 bf16, 1 fp16
  int64_t B, H, Hkv, Sq, Sk, d;
  TokMap qmap, kmap;  // row offsets of q and k
  double* partial;  // fp4i_balance_partials doubles
  int32_t* exps;    // [B, Hkv, d]
};
size_t fp4i_balance_partials(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t d);
hipError_t fp4i_launch_balance(const BalanceLaunch& L, hipStream_t stream);

int fp4i_amax_parts(int64_t rows, int64_t cols);
hipError_t fp4i_launch_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int axis,
                                   uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t fp4i_launch_quantize(const QuantLaunch& L, hipStream_t stream);
// Q and K (axis 0) and V (axis 1) in one launch; only for gmode 0 with no
// per-tensor scale, rotation, balance exponents or block means, bf16/fp16
// (hipErrorInvalidValue otherwise).  Same results as three fp4i_launch_quantize.
hipError_t fp4i_launch_quantize_qkv(const QuantLaunch& q, const QuantLaunch& k, const QuantLaunch& v,
                                    hipStream_t stream);

// MXFP4 attention forward: Q, K codes [.., d/2] with E8M0 scales [.., d/32]
// (blocks along d), V codes [.., Sk/2, d] with scales [.., Sk/32, d] (blocks
// along tokens); Sk % 32 == 0.
struct MxAttnLaunch {
  int64_t B, H, Hkv, Sq, Sk, d;
  const uint8_t *qc, *qs, *kc, *ks, *vc, *vs;
  int causal;
  float c;  // log2(e) * softmax_scale
  int kv_tile;
  int out_dtype;
  void* out;
  float* lse;
};
hipError_t fp4i_launch_attn_mx(const MxAttnLaunch& L, hipStream_t stream);

struct TopkLaunch {
  const void* q;  // [B,H,Sq,d]
  const void* k;  // [B,Hkv,Sk,d]
  int dtype;
  int64_t B, H, Hkv, Sq, Sk, d;
  int causal, pct, sel_block;
  int nqb, nkb, kmax;
  double* qmeans;  // [B*H, nqb, d]
  double* kmeans;  // [B*Hkv, nkb, d]
  int means_ready = 0;  // 1: the quantizer already wrote both
  TokMap qmap, kmap;    // row offsets of q and k (for the means)
  uint64_t* keys;  // [B*H, nqb, nkb] order-preserving keys of the block scores
  int32_t* idx;    // [B*H, nqb, kmax]
  int32_t* cnt;    // [B*H, nqb]
};

hipError_t fp4i_launch_topk(const TopkLaunch& L, hipStream_t stream);

struct AttnLaunch {
  int64_t B, H, Hkv, Sq, Sk, d;
  int dtype;  // of q, k, v (0 bf16, 1 fp16)
  const void* q;
  const void* k;
  const void* v;
  TokMap qmap, kmap, vmap;  // row offsets of q, k, v (the FP16 path reads them)
  int strided = 0;          // some of them is not dense
  const uint8_t* qc;
  const uint8_t* qs;
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  int causal;
  float c;  // log2(e) * softmax_scale, rounded once to binary32
  int kv_tile;
  int pct, sel_block, nqb, kmax;
  int p_mode;          // P on the FP4 tiles: 0 two-level, 1 single-level, 2 unquantized (O')
  const int32_t* idx;  // selection (pct > 0)
  const int32_t* cnt;
  int out_dtype;
  void* out;
  float* lse;
};

hipError_t fp4i_launch_attn_fwd(const AttnLaunch& L, hipStream_t stream);

// Backward of the FP4 attention (training).
struct AttnBwdLaunch {
  int64_t B, H, Hkv, Sq, Sk, d;
  int dtype;       // of dout (0 bf16, 1 fp16)
  int hp_dtype;    // of out_hp (0 bf16, 1 fp16, 2 fp32)
  const uint8_t *qc, *qs, *kc, *ks, *vc, *vs;
  const void* dout;
  const void* out_hp;
  const float* lse;
  int causal, kv_tile, single;
  float c;
  float *dq, *dk, *dv;
  void* ws;
};

size_t fp4i_attn_bwd_workspace(const AttnBwdLaunch& L);
hipError_t fp4i_launch_attn_bwd(const AttnBwdLaunch& L, hipStream_t stream);

struct DecodeLaunch {
  const void* q;  // bf16 [B,Hq,d]
  int64_t B, Hq, Hkv, d;
  int n_sink, n_recent;
  int64_t mid_cap;
  const void* k_sink;
  const void* v_sink;
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  const void* k_recent;
  const void* v_recent;
  const int32_t* mid_len;
  float c;  // log2(e) * softmax_scale
  int out_dtype;
  void* out;
  float* lse;
  int nsplit;        // context splits per (b, kv head)
  int nfull;         // full-precision (sink + recent) workgroups per (b, kv head)
  int64_t split_len; // tokens per split of the FP4 region (multiple of the chunk)
  float* part_o;     // [B*Hq, nsplit+nfull+nprom, d]
  float* part_ml;    // [B*Hq, nsplit+nfull+nprom, 2]
  // selective promotion (nprom = 0: none)
  const void* k_mid;         // bf16 [B,Hkv,mid_cap,d]
  const void* v_mid;
  const int32_t* sel_idx;    // [B*Hkv, kmax]
  const uint32_t* sel_mask;  // [B*Hkv, nbw] bit j: middle block j promoted
  int kmax, nprom, nbw;      // nprom = ceil(kmax / 4) workgroups of promoted blocks
};

int fp4i_decode_splits(int64_t B, int64_t Hkv, int64_t mid_cap, int64_t* split_len);

// Selection of the promoted middle blocks for decode.
struct DecSelectLaunch {
  const void* q;         // bf16 [B,Hq,d]
  const double* k_sum;   // [B*Hkv, nbc, d]
  const int32_t* mid_len;
  int64_t B, Hq, Hkv, d, mid_cap;
  int pct, kmax, nbc, nbw;
  uint64_t* keys;        // [B*Hkv, nbc] workspace
  int32_t* idx;          // [B*Hkv, kmax]
  int32_t* cnt;          // [B*Hkv]
  uint32_t* mask;        // [B*Hkv, nbw]
};

constexpr int kDecSelBlock = 128;  // tokens per selection block of the middle
hipError_t fp4i_launch_decode_select(const DecSelectLaunch& L, hipStream_t stream);
hipError_t fp4i_launch_kv_block_sums(const void* k_mid, const int32_t* mid_len, double* k_sum, int64_t B,
                                     int64_t Hkv, int64_t mid_cap, int64_t d, hipStream_t stream);

struct KvAppendLaunch {
  int64_t B, Hkv, d, mid_cap;
  int n_recent, n_new;
  const void* k_new;  // bf16 [B,Hkv,n_new,d]
  const void* v_new;
  void* k_recent;     // bf16 [B,Hkv,n_recent,d]
  void* v_recent;
  uint8_t *kc, *ks, *vc, *vs;
  int32_t* mid_len;
  int32_t* overflow;  // nullable
  void* ws;
  void* k_mid;        // full-precision copy of the middle (nullable, with v_mid and k_sum)
  void* v_mid;
  double* k_sum;
};

size_t fp4i_kv_append_workspace(int64_t B, int64_t Hkv, int64_t n_recent, int64_t d);
hipError_t fp4i_launch_kv_append(const KvAppendLaunch& L, hipStream_t stream);
int fp4i_decode_full_splits(int64_t n_full);
hipError_t fp4i_launch_decode(const DecodeLaunch& L, hipStream_t stream);

// Sets the thread's fp4_last_error message and returns code (api.cpp).
int fp4i_fail(int code, const char* msg);

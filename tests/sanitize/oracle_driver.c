/* Runs every C entry point of the oracle on small inputs; built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py.
 * Any out-of-bounds access, leak or undefined operation aborts the run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t orc_quantize(const float* x, int64_t rows, int64_t cols, int block_axis, int scale_search, int fmin,
                     int fmax, int global_mode, float* g_io, uint8_t* codes, uint8_t* scales, int8_t* offsets);
void orc_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, int block_axis,
                    float g, double* out);
void orc_hadamard_rows(float* x, int64_t rows, int n, const uint32_t* signs);
void orc_block_means(const float* x, int64_t S, int d, int blk, double* means);
void orc_block_sums(const float* x, int64_t S, int d, int blk, double* sums);
void orc_block_topk(const double* qm, const double* km, int nqb, int nkb, int d, int causal, int pct, int kmax,
                    int32_t* idx, int32_t* cnt);
int orc_topk_count(int pct, int n);
void orc_mx_quantize(const float* x, int64_t rows, int64_t cols, int block_axis, uint8_t* codes, uint8_t* scales);
void orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, int block_axis,
                       double* out);
int orc_attention_fwd(const float* q, const float* k, const float* v, int B, int H, int Hkv, int64_t Sq, int64_t Sk,
                      int d, int causal, double softmax_scale, int kv_tile, int scale_search, int fmin, int fmax,
                      int pct, int sel_block, const int64_t* rows, int64_t n_rows, const int* heads, int n_heads,
                      float* out, float* lse, int32_t* topk_idx, int32_t* topk_cnt, const float* q_fp4,
                      const float* k_fp4, int single_level, double* probs, double* probs_hat, int mx,
                      const double* tie, double* amb);
int orc_attention_exact(const float* q, const float* k, const float* v, int B, int H, int Hkv, int64_t Sq,
                        int64_t Sk, int d, int causal, double softmax_scale, const int64_t* rows, int64_t n_rows,
                        const int* heads, int n_heads, float* out, float* lse);
int orc_attention_decode(const float* q, const float* k, const float* v, const int32_t* ctx_len, int B, int Hq,
                         int Hkv, int d, int64_t Lcap, int n_sink, int n_recent, double softmax_scale,
                         int scale_search, int fmin, int fmax, const int* pairs, int n_pairs, float* out, float* lse,
                         int pct, int sel_blk, int kmax, int32_t* sel_idx, int32_t* sel_cnt);

static uint64_t state = 0x9E3779B97F4A7C15ull;

static float gauss(void) {  /* sum of four uniforms, centred: enough spread for these checks */
  float s = 0.0f;
  for (int i = 0; i < 4; ++i) {
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    s += (float)((state >> 40) & 0xFFFFFF) / 16777216.0f;
  }
  return (s - 2.0f) * 1.7f;
}

static float* randn(int64_t n) {
  float* x = malloc(sizeof(float) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) x[i] = gauss();
  return x;
}

#define CHECK(c)                                            \
  do {                                                      \
    if (!(c)) {                                             \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                             \
    }                                                       \
  } while (0)

int main(void) {
  /* quantizer, both axes, with and without the search, per-tensor scale */
  const int64_t R = 48, Cc = 64;
  float* x = randn(R * Cc);
  x[5] = 40.0f;
  uint8_t* codes = calloc((size_t)(R * Cc / 2), 1);
  uint8_t* scales = calloc((size_t)(R * Cc / 16), 1);
  int8_t* offs = calloc((size_t)(R * Cc / 16), 1);
  double* deq = malloc(sizeof(double) * (size_t)(R * Cc));
  for (int axis = 0; axis < 2; ++axis)
    for (int gm = 0; gm < 3; ++gm) {
      float g = 0.05f;
      CHECK(orc_quantize(x, R, Cc, axis, 1, -2, 6, gm, &g, codes, scales, offs) >= 0);
      orc_dequantize(codes, scales, R, Cc, axis, g, deq);
      CHECK(orc_quantize(x, R, Cc, axis, 0, 0, 0, gm, &g, codes, scales, NULL) >= 0);
    }
  /* rotation, means, sums, selection */
  const uint32_t signs[4] = {0x12345678u, 0x9ABCDEF0u, 0x0F0F0F0Fu, 0xF0F0F0F0u};
  orc_hadamard_rows(x, R, 64, signs);
  orc_hadamard_rows(x, R, 16, NULL);
  double* qm = malloc(sizeof(double) * 4 * 64);
  double* km = malloc(sizeof(double) * 4 * 64);
  orc_block_means(x, R, 64, 16, qm);
  orc_block_sums(x, R, 64, 16, km);
  int kmax = orc_topk_count(50, 3);
  int32_t idx[3 * 4], cnt[3];
  orc_block_topk(qm, km, 3, 3, 64, 1, 50, kmax, idx, cnt);
  /* MXFP4 */
  orc_mx_quantize(x, R, Cc, 0, codes, scales);
  orc_mx_dequantize(codes, scales, R, Cc, 0, deq);
  orc_mx_quantize(x, R - 16, Cc, 1, codes, scales);
  orc_mx_dequantize(codes, scales, R - 16, Cc, 1, deq);
  /* attention: ragged tiles, GQA, selection, probabilities, single-level and MX P */
  const int B = 1, H = 2, Hkv = 1, d = 64;
  const int64_t S = 160;
  float* q = randn(B * H * S * d);
  float* k = randn(B * Hkv * S * d);
  float* v = randn(B * Hkv * S * d);
  float* out = malloc(sizeof(float) * (size_t)(B * H * S * d));
  float* lse = malloc(sizeof(float) * (size_t)(B * H * S));
  double* probs = malloc(sizeof(double) * (size_t)(B * H * S * S));
  double* probs_hat = malloc(sizeof(double) * (size_t)(B * H * S * S));
  int32_t tidx[2 * 2 * 2], tcnt[2 * 2];
  const double tie[2] = {1e-6, 1e-7};
  double* amb = malloc(sizeof(double) * (size_t)(B * H * S));
  CHECK(orc_attention_fwd(q, k, v, B, H, Hkv, S, S, d, 1, 0.0, 64, 1, -2, 6, 50, 128, NULL, 0, NULL, 0, out, lse,
                          tidx, tcnt, NULL, NULL, 0, NULL, NULL, 0, tie, amb) == 0);
  CHECK(orc_attention_fwd(q, k, v, B, H, Hkv, S, S, d, 0, 0.0, 128, 1, -2, 6, 0, 128, NULL, 0, NULL, 0, out, lse,
                          NULL, NULL, NULL, NULL, 1, probs, probs_hat, 0, tie, amb) == 0);
  CHECK(orc_attention_fwd(q, k, v, B, H, Hkv, S, S, d, 1, 0.0, 64, 0, 0, 0, 0, 128, NULL, 0, NULL, 0, out, lse,
                          NULL, NULL, NULL, NULL, 0, NULL, NULL, 1, NULL, NULL) == 0);
  const int64_t rows[3] = {0, 77, 159};
  const int heads[1] = {1};
  CHECK(orc_attention_fwd(q, k, v, B, H, Hkv, S, S, d, 1, 0.2, 128, 1, -2, 6, 0, 128, rows, 3, heads, 1, out, lse,
                          NULL, NULL, NULL, NULL, 0, NULL, NULL, 0, NULL, NULL) == 0);
  CHECK(orc_attention_exact(q, k, v, B, H, Hkv, S, S, d, 1, 0.0, rows, 3, NULL, 0, out, lse) == 0);
  /* decode over a cache with sink, middle and recent tokens, with and without promotion */
  const int Bd = 2, Hq = 4, Hk = 2;
  const int64_t L = 256;
  float* dq = randn(Bd * Hq * d);
  float* dk = randn(Bd * Hk * L * d);
  float* dv = randn(Bd * Hk * L * d);
  int32_t ctx[2] = {256, 208};
  float* dout = malloc(sizeof(float) * (size_t)(Bd * Hq * d));
  float* dlse = malloc(sizeof(float) * (size_t)(Bd * Hq));
  int32_t sidx[2 * 2 * 2], scnt[2 * 2];
  CHECK(orc_attention_decode(dq, dk, dv, ctx, Bd, Hq, Hk, d, L, 16, 32, 0.0, 1, -2, 6, NULL, 0, dout, dlse, 0, 64,
                             0, NULL, NULL) == 0);
  CHECK(orc_attention_decode(dq, dk, dv, ctx, Bd, Hq, Hk, d, L, 16, 32, 0.0, 1, -2, 6, NULL, 0, dout, dlse, 50, 64,
                             2, sidx, scnt) == 0);
  /* rejected arguments */
  CHECK(orc_quantize(x, R, 40, 0, 1, -2, 6, 0, NULL, codes, scales, NULL) < 0);
  CHECK(orc_attention_fwd(q, k, v, B, H, Hkv, S, S, d, 1, 0.0, 48, 0, 0, 0, 0, 128, NULL, 0, NULL, 0, out, lse,
                          NULL, NULL, NULL, NULL, 0, NULL, NULL, 1, NULL, NULL) != 0);
  free(x); free(codes); free(scales); free(offs); free(deq); free(qm); free(km);
  free(q); free(k); free(v); free(out); free(lse); free(probs); free(probs_hat); free(amb);
  free(dq); free(dk); free(dv); free(dout); free(dlse);
  printf("oracle driver ok\n");
  return 0;
}

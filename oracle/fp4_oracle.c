/*
 * fp4_oracle.c -- plain, slow CPU oracle for block-scaled FP4 (E2M1 elements,
 * E4M3 block scales over 16 elements) quantization and FP4 attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * tables or constants with the GPU library; the two are written independently
 * from the same definitions.
 *
 * Sources (web pages, cited by title and section):
 *   [ScaleSearch]  "Busca tus escalas de punto flotante por bloques" summary:
 *                  Declaracion del Problema (NVFP4 = E2M1 + 8-bit E4M3 scale),
 *                  Metodologia / ScaleSearch (max scaling, integer offset on the
 *                  scale's bit pattern, MSE search), Metodologia /
 *                  ScaleSearchAttention (QK^T and PV on NVFP4 with FP32
 *                  accumulation; sink-aware KV cache precision).
 *   [Thrift]       "ThriftAttention" summary: Metodologia / 1 (block means,
 *                  score = dot product of means, top-k) and 2 (FP16 path for
 *                  the selected pairs, FP4 path for the rest, online-softmax
 *                  fusion, two-level quantization of P).
 *   [AttnQAT]      "Attn-QAT" summary: Resumo tecnico / 1 (FP4 has 15 distinct
 *                  values).
 *
 * Where the pages leave a step open, the reading used here is stated at the
 * step.  Floating point is IEEE binary32 where the method fixes a decision
 * (codes, scales, offsets) and binary64 elsewhere.  Build with
 * -ffp-contract=off so that no multiply-add is fused.
 *
 * Parity status: every function here is pinned by CPU tests against closed
 * forms, exact-rational brute force, invariants or textbook references.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* E2M1 magnitudes: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
   Seven non-zero magnitudes, so with the sign there are 15 distinct values
   ([AttnQAT] Resumo tecnico / 1). */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int code) {
  double m = kE2M1[code & 7];
  return (code & 8) ? -m : m;
}

/* E4M3 (OCP "FN" variant, bias 7): exponent field 0 is subnormal m/8 * 2^-6,
   otherwise (1 + m/8) * 2^(e-7); 0x7F and 0xFF are NaN, so the largest finite
   value is 0x7E = 448.  Scale bytes never carry a sign ([ScaleSearch] writes
   the scale type as unsigned E4M3). */
double orc_e4m3_value(int byte) {
  int e = (byte >> 3) & 15, m = byte & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return (byte & 0x80) ? -v : v;
}

/* Nearest non-negative E4M3 byte (0..0x7E) to v >= 0; on a tie the byte with
   an even mantissa (even byte value) wins.  Values above 448 go to 448
   (saturation: 448 is nearest), never to NaN. */
int orc_e4m3_encode(double v) {
  if (v >= 448.0) return 0x7E; /* saturation (also keeps huge v out of the distance test) */
  int best = 0;
  double bd = fabs(v);
  for (int b = 1; b <= 0x7E; ++b) {
    double dd = fabs(v - orc_e4m3_value(b));
    if (dd < bd || (dd == bd && (b & 1) == 0)) { bd = dd; best = b; }
  }
  return best;
}

/* Nearest E2M1 magnitude code (0..7) to t >= 0; ties go to the even code
   (0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4); t > 6 gives 6. */
int orc_e2m1_encode(double t) {
  if (t >= 6.0) return 7; /* saturation: for huge t the binary64 distances would tie */
  int best = 0;
  double bd = fabs(t);
  for (int c = 1; c < 8; ++c) {
    double dd = fabs(t - kE2M1[c]);
    if (dd < bd || (dd == bd && (c & 1) == 0)) { bd = dd; best = c; }
  }
  return best;
}

/* Correctly rounded binary32 reciprocal of a positive scale byte. */
float orc_recip(int byte) {
  float s = (float)orc_e4m3_value(byte);
  return 1.0f / s;
}

/* binary16 round-to-nearest-even of a double (result returned as double). */
double orc_round_fp16(double x) {
  if (x == 0.0 || isnan(x)) return x;
  double ax = fabs(x);
  int e;
  frexp(ax, &e);              /* ax = f * 2^e, f in [0.5,1) */
  int ulp_exp = e - 11;       /* 11 significant bits */
  if (ulp_exp < -24) ulp_exp = -24;  /* subnormal spacing 2^-24 */
  double q = ldexp(ax, -ulp_exp);
  double r = nearbyint(q);    /* default rounding mode: nearest, ties even */
  double y = ldexp(r, ulp_exp);
  if (y > 65504.0) y = INFINITY;
  return x < 0 ? -y : y;
}

/* ------------------------------------------------------------------------ */
/* Block quantization ([ScaleSearch] Metodologia / ScaleSearch)              */
/* ------------------------------------------------------------------------ */

/* Squared error of one 16-element block (values y, already in the scaled
   domain) quantized with scale byte b.  Reading of the pages' MSE: binary32,
   element error |y| - v(c)*s (the product is exact), squared, then summed in
   a fixed pairwise tree (0+1, 2+3, ... then pairs of pairs).  Scale byte 0
   means every code is zero.  Elements are mapped to the grid by multiplying
   |y| with the correctly rounded reciprocal of the scale and rounding to the
   nearest E2M1 value (ties to even). */
static float block_sse(const float* ay, int b, uint8_t* mag_out) {
  float q[16];
  if (b == 0) {
    for (int k = 0; k < 16; ++k) {
      q[k] = ay[k] * ay[k];
      if (mag_out) mag_out[k] = 0;
    }
  } else {
    float s = (float)orc_e4m3_value(b);
    float r = orc_recip(b);
    for (int k = 0; k < 16; ++k) {
      float t = ay[k] * r;
      int c = orc_e2m1_encode((double)t);
      float deq = (float)kE2M1[c] * s; /* exact: at most 6 significant bits */
      float e = ay[k] - deq;
      q[k] = e * e;
      if (mag_out) mag_out[k] = (uint8_t)c;
    }
  }
  float l1[8], l2[4], l3[2];
  for (int k = 0; k < 8; ++k) l1[k] = q[2 * k] + q[2 * k + 1];
  for (int k = 0; k < 4; ++k) l2[k] = l1[2 * k] + l1[2 * k + 1];
  for (int k = 0; k < 2; ++k) l3[k] = l2[2 * k] + l2[2 * k + 1];
  return l3[0] + l3[1];
}

/* Quantize one block of 16 binary32 values y[k*stride].
   Steps: a = max|y|; max-scaling scale s0 = E4M3(a/6) (the division is
   binary32, correctly rounded, then rounded to the nearest E4M3 value, ties
   to even, saturating at 448); ScaleSearch adds an integer offset f to the
   scale's bit pattern for f in [fmin, fmax] (candidates whose byte leaves
   0..0x7E are skipped) and keeps the candidate of least squared error, the
   lowest f on ties.  Without ScaleSearch only f = 0 is tried.
   Outputs: 16 unpacked codes (sign bit 3 copied from y), the scale byte and
   the chosen offset.  A block holding Inf or NaN gets scale byte 0x7F, zero
   codes, and the function returns 1; otherwise 0.
   sse_out (nullable) receives the error of every candidate f (NaN where the
   candidate is invalid). */
int orc_quantize_block(const float* y, int stride, int scale_search, int fmin, int fmax,
                       uint8_t* codes, uint8_t* scale, int8_t* off, float* sse_out) {
  float ay[16];
  float a = 0.0f;
  int nonfinite = 0;
  for (int k = 0; k < 16; ++k) {
    float v = y[(int64_t)k * stride];
    if (!isfinite(v)) nonfinite = 1;
    ay[k] = fabsf(v);
    if (ay[k] > a) a = ay[k];
  }
  if (sse_out)
    for (int f = fmin; f <= fmax; ++f) sse_out[f - fmin] = NAN;
  if (nonfinite) {
    for (int k = 0; k < 16; ++k) codes[k] = signbit(y[(int64_t)k * stride]) ? 8 : 0;
    *scale = 0x7F;
    *off = 0;
    return 1;
  }
  if (a == 0.0f) {
    for (int k = 0; k < 16; ++k) codes[k] = signbit(y[(int64_t)k * stride]) ? 8 : 0;
    *scale = 0;
    *off = 0;
    return 0;
  }
  float a6 = a / 6.0f;
  int s0 = orc_e4m3_encode((double)a6);
  int lo = scale_search ? fmin : 0, hi = scale_search ? fmax : 0;
  int best_f = 0, have = 0;
  float best = 0.0f;
  for (int f = lo; f <= hi; ++f) {
    int b = s0 + f;
    if (b < 0 || b > 0x7E) continue;
    float e = block_sse(ay, b, NULL);
    if (sse_out) sse_out[f - fmin] = e;
    if (!have || e < best) { best = e; best_f = f; have = 1; }
  }
  uint8_t mag[16];
  int b = s0 + best_f;
  block_sse(ay, b, mag);
  for (int k = 0; k < 16; ++k) {
    int sgn = signbit(y[(int64_t)k * stride]) ? 8 : 0;
    codes[k] = (uint8_t)(mag[k] | sgn);
  }
  *scale = (uint8_t)b;
  *off = (int8_t)best_f;
  return 0;
}

/* Per-tensor scale (reading: the optional second level of NVFP4 is one
   binary32 decode scale g = amax/2688 with 2688 = 6 * 448, the largest value an
   element times a scale can take; elements are first multiplied by the
   correctly rounded 2688/amax).  mode 0: g = 1.  mode 1: computed from the
   tensor (NaN ignored; an all-zero tensor gives g = 1).  mode 2: g given in
   *g_io, the encode factor is 1/g. */
static void global_scale(const float* x, int64_t n, int mode, float* g_io, float* ginv) {
  if (mode == 0) { *g_io = 1.0f; *ginv = 1.0f; return; }
  if (mode == 2) { *ginv = 1.0f / *g_io; return; }
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float v = fabsf(x[i]);
    if (v > amax) amax = v; /* NaN compares false: ignored */
  }
  if (amax == 0.0f) { *g_io = 1.0f; *ginv = 1.0f; return; }
  *g_io = amax / 2688.0f;
  *ginv = 2688.0f / amax;
}

/* Quantize a dense row-major [rows, cols] binary32 tensor.
   block_axis 0: blocks are 16 consecutive columns of a row; codes are
     [rows][cols/2] (element 2i in the low nibble), scales/offsets [rows][cols/16].
   block_axis 1: blocks are 16 consecutive rows of a column; codes are
     [rows/2][cols] (row 2i in the low nibble), scales/offsets [rows/16][cols].
   Returns the number of blocks holding Inf/NaN, or -1 on bad arguments. */
int64_t orc_quantize(const float* x, int64_t rows, int64_t cols, int block_axis, int scale_search,
                     int fmin, int fmax, int global_mode, float* g_io, uint8_t* codes,
                     uint8_t* scales, int8_t* offsets) {
  if (block_axis == 0 && cols % 16) return -1;
  if (block_axis == 1 && rows % 16) return -1;
  float ginv;
  global_scale(x, rows * cols, global_mode, g_io, &ginv);
  int64_t nb = rows * cols / 16;
  int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (int64_t blk = 0; blk < nb; ++blk) {
    float y[16];
    int64_t r0, c0;
    if (block_axis == 0) { r0 = blk / (cols / 16); c0 = (blk % (cols / 16)) * 16; }
    else { r0 = (blk / cols) * 16; c0 = blk % cols; }
    for (int k = 0; k < 16; ++k) {
      int64_t r = block_axis == 0 ? r0 : r0 + k, c = block_axis == 0 ? c0 + k : c0;
      float v = x[r * cols + c];
      y[k] = global_mode == 0 ? v : v * ginv;
    }
    uint8_t cd[16], sc;
    int8_t of;
    bad += orc_quantize_block(y, 1, scale_search, fmin, fmax, cd, &sc, &of, NULL);
    for (int k = 0; k < 16; ++k) {
      int64_t r = block_axis == 0 ? r0 : r0 + k, c = block_axis == 0 ? c0 + k : c0;
      int64_t byte_idx, shift;
      if (block_axis == 0) { byte_idx = r * (cols / 2) + c / 2; shift = (c & 1) * 4; }
      else { byte_idx = (r / 2) * cols + c; shift = (r & 1) * 4; }
      if (shift == 0) codes[byte_idx] = (uint8_t)((codes[byte_idx] & 0xF0) | cd[k]);
      else codes[byte_idx] = (uint8_t)((codes[byte_idx] & 0x0F) | (cd[k] << 4));
    }
    int64_t si = block_axis == 0 ? r0 * (cols / 16) + c0 / 16 : (r0 / 16) * cols + c0;
    scales[si] = sc;
    if (offsets) offsets[si] = of;
  }
  return bad;
}

/* Dequantize to binary64: value = v(code) * scale * g (exact in binary64). */
void orc_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                    int block_axis, float g, double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      int code;
      int sc;
      if (block_axis == 0) {
        uint8_t byte = codes[r * (cols / 2) + c / 2];
        code = (c & 1) ? byte >> 4 : byte & 15;
        sc = scales[r * (cols / 16) + c / 16];
      } else {
        uint8_t byte = codes[(r / 2) * cols + c];
        code = (r & 1) ? byte >> 4 : byte & 15;
        sc = scales[(r / 16) * cols + c];
      }
      out[r * cols + c] = orc_e2m1_value(code) * orc_e4m3_value(sc) * (double)g;
    }
}

/* ------------------------------------------------------------------------ */
/* Incoherence processing ([ScaleSearch] Metodologia / ScaleSearchAttention:  */
/* Hadamard transforms of Q and K before quantization)                       */
/* ------------------------------------------------------------------------ */

/* Each row v of x [rows][n] (n a power of two) becomes H_n (s o v) / sqrt(n):
   s_j = -1 where bit j of signs (32 bits per word) is set, else +1 (the sign
   flip is exact); H_n is the Sylvester Hadamard matrix, applied by butterfly
   stages of span h = 1, 2, 4, ..., n/2, each pair (i, i+h) with bit h of i
   clear becoming (a + b, a - b) in binary32; then every element is
   multiplied by the binary32 value of 1/sqrt(n).  The rotation R =
   diag(s) H_n / sqrt(n) is orthogonal, so (Q R)(K R)^T = Q K^T. */
void orc_hadamard_rows(float* x, int64_t rows, int n, const uint32_t* signs) {
  const float c = (float)(1.0 / sqrt((double)n));
  for (int64_t r = 0; r < rows; ++r) {
    float* v = x + r * n;
    for (int j = 0; j < n; ++j)
      if (signs && ((signs[j >> 5] >> (j & 31)) & 1u)) v[j] = -v[j];
    for (int h = 1; h < n; h <<= 1)
      for (int i = 0; i < n; ++i)
        if (!(i & h)) {
          float a = v[i], b = v[i + h];
          v[i] = a + b;
          v[i + h] = a - b;
        }
    for (int j = 0; j < n; ++j) v[j] = v[j] * c;
  }
}

/* Magnitude balance of Q and K (ScaleSearch page, Metodologia /
   ScaleSearchAttention: besides the Hadamard rotation, a pair Q' = Q R^-T,
   K' = K R keeps the scores Q K^T and lowers the mean squared magnitude of the
   two tensors).  Reading: R is diagonal with power-of-two entries 2^e_c, one
   vector per (batch, kv head), fitted to the call's own Q and K: with ms_q[c]
   the mean of q^2 over the group's query heads and all query tokens and
   ms_k[c] the mean of k^2 over the kv head's tokens (binary64 sums in
   ascending head then token order, divided by the count), e_c is the integer
   in [-8, 8] minimizing ms_q 4^-e + ms_k 4^e: the smallest e with
   4^(2e+1) >= ms_q / ms_k (ties go to the lower e).  A channel whose mean
   square is 0 on either side keeps e = 0.  Then Q'_c = Q_c 2^-e_c and
   K'_c = K_c 2^e_c are exact in binary32 (away from overflow and underflow)
   and Q' K'^T = Q K^T.  e: [B][Hkv][d]. */
void orc_balance_exponents(const float* q, const float* k, int B, int H, int Hkv, int64_t Sq, int64_t Sk, int d,
                           int32_t* e) {
  const int G = H / Hkv;
  for (int b = 0; b < B; ++b)
    for (int hk = 0; hk < Hkv; ++hk)
      for (int c = 0; c < d; ++c) {
        double sq = 0.0, sk = 0.0;
        for (int g = 0; g < G; ++g) {
          const float* qh = q + (((int64_t)b * H + hk * G + g) * Sq) * d;
          for (int64_t t = 0; t < Sq; ++t) sq += (double)qh[t * d + c] * (double)qh[t * d + c];
        }
        const float* kh = k + (((int64_t)b * Hkv + hk) * Sk) * d;
        for (int64_t t = 0; t < Sk; ++t) sk += (double)kh[t * d + c] * (double)kh[t * d + c];
        const double mq = sq / (double)(G * Sq), mk = sk / (double)Sk;
        int ec = 0;
        if (mq > 0.0 && mk > 0.0) {
          const double A = mq / mk;
          ec = 8;
          for (int x = -8; x <= 8; ++x)
            if (ldexp(1.0, 2 * (2 * x + 1)) >= A) { ec = x; break; }
        }
        e[((int64_t)b * Hkv + hk) * d + c] = ec;
      }
}

/* ------------------------------------------------------------------------ */
/* Block selection ([Thrift] Metodologia / 1)                                */
/* ------------------------------------------------------------------------ */

/* Mean vector of each block of `blk` consecutive tokens of x [S][d]; the sum
   runs over ascending tokens in binary64, then divides by the token count. */
void orc_block_means(const float* x, int64_t S, int d, int blk, double* means) {
  int64_t nb = (S + blk - 1) / blk;
  for (int64_t ib = 0; ib < nb; ++ib) {
    int64_t t0 = ib * blk, t1 = t0 + blk < S ? t0 + blk : S;
    for (int c = 0; c < d; ++c) {
      double s = 0.0;
      for (int64_t t = t0; t < t1; ++t) s += (double)x[t * d + c];
      means[ib * d + c] = s / (double)(t1 - t0);
    }
  }
}

/* Sum of each block of `blk` consecutive tokens of x [S][d] (the last block
   may be short), in binary64 over ascending tokens: the numerators of
   orc_block_means, kept by a cache so that appends can extend them. */
void orc_block_sums(const float* x, int64_t S, int d, int blk, double* sums) {
  int64_t nb = (S + blk - 1) / blk;
  for (int64_t ib = 0; ib < nb; ++ib) {
    int64_t t0 = ib * blk, t1 = t0 + blk < S ? t0 + blk : S;
    for (int c = 0; c < d; ++c) {
      double s = 0.0;
      for (int64_t t = t0; t < t1; ++t) s += (double)x[t * d + c];
      sums[ib * d + c] = s;
    }
  }
}

/* Number of selected key blocks for a query block that sees n key blocks:
   ceil(pct * n / 100) in integers. */
int orc_topk_count(int pct, int n) { return (pct * n + 99) / 100; }

/* Score of a block pair: the binary64 dot product of the two block means,
   one fused multiply-add per channel in ascending channel order (each step
   is the exact s + q_c k_c rounded once; the page fixes the dot product, not
   its rounding). */
static double block_score(const double* q, const double* k, int d) {
  double s = 0.0;
  for (int c = 0; c < d; ++c) s = fma(q[c], k[c], s);
  return s;
}

/* Every score of query blocks x key blocks (out [nqb, nkb]). */
void orc_block_scores(const double* qm, const double* km, int nqb, int nkb, int d, double* out) {
  for (int i = 0; i < nqb; ++i)
    for (int j = 0; j < nkb; ++j) out[(int64_t)i * nkb + j] = block_score(qm + (int64_t)i * d, km + (int64_t)j * d, d);
}

/* For every query block i: score each visible key block j (j <= i when
   causal), keep the k_i highest (ties: lower j first), and write them in
   ascending j order, padded with -1 to kmax entries. */
void orc_block_topk(const double* qm, const double* km, int nqb, int nkb, int d, int causal,
                    int pct, int kmax, int32_t* idx, int32_t* cnt) {
  double* sc = (double*)malloc(sizeof(double) * (size_t)nkb);
  char* taken = (char*)malloc((size_t)nkb);
  for (int i = 0; i < nqb; ++i) {
    int nvis = causal ? (i + 1 < nkb ? i + 1 : nkb) : nkb;
    for (int j = 0; j < nvis; ++j) {
      sc[j] = block_score(qm + (int64_t)i * d, km + (int64_t)j * d, d);
      taken[j] = 0;
    }
    int k = orc_topk_count(pct, nvis);
    for (int r = 0; r < k; ++r) {
      int bj = -1;
      for (int j = 0; j < nvis; ++j) {
        if (taken[j]) continue;
        if (bj < 0 || sc[j] > sc[bj]) bj = j; /* strict: the lower j keeps ties */
      }
      taken[bj] = 1;
    }
    int w = 0;
    for (int j = 0; j < nvis; ++j)
      if (taken[j]) idx[(int64_t)i * kmax + w++] = j;
    for (; w < kmax; ++w) idx[(int64_t)i * kmax + w] = -1;
    cnt[i] = k;
  }
  free(sc);
  free(taken);
}

/* ------------------------------------------------------------------------ */
/* FP4 attention, fake-quant numerics                                        */
/* ------------------------------------------------------------------------ */

/* exp2 rounded once to binary32 (reading: the pages leave exp unspecified;
   the plain definition is the correctly rounded 2^z). */
static float exp2_f32(float z) { return (float)exp2((double)z); }

/* Conversion factor from softmax scale to base-2 exponent, computed in
   binary64 and rounded once: c = log2(e) * scale, scale = 1/sqrt(d) by default. */
float orc_score_factor(double softmax_scale, int d) {
  double s = softmax_scale > 0.0 ? softmax_scale : 1.0 / sqrt((double)d);
  return (float)(1.4426950408889634074 * s);
}

typedef struct {
  double* O;     /* [d] */
  double l;      /* sum of unquantized e */
  float tm;      /* tile-row maximum of x */
  int fp4;       /* 1: FP4 path (O in units of 2688), 0: FP16 path */
} tile_acc;

/* Quantize a dense [S][d] slice and return its binary64 dequantized copy. */
/* ------------------------------------------------------------------------ */
/* MXFP4: E2M1 elements with one power-of-two (E8M0) scale per 32 elements,  */
/* the classic block floating point the ScaleSearch page contrasts NVFP4     */
/* with (Declaracion del Problema: a scale fixed by the block maximum, no    */
/* mantissa bits).  Scale rule of the OCP microscaling format: shared        */
/* exponent floor(log2(amax)) - 2 (2 = the exponent of E2M1's largest value),*/
/* elements rounded to nearest E2M1 (ties to the even code) with saturation  */
/* at 6 -- values in [6, 8) times the scale clip to 6.                       */
/* ------------------------------------------------------------------------ */

/* Scale byte (biased by 127) of a block with maximum magnitude a, the
   shared exponent clamped to [-127, 127]; 0 for a = 0 (every code is then
   0), 0xFF for a non-finite maximum. */
int orc_mx_scale_byte(double a) {
  if (!(a == a) || a == INFINITY) return 0xFF;
  if (a == 0.0) return 0;
  int ex;
  frexp(a, &ex);            /* a = m 2^ex, m in [0.5, 1): floor(log2 a) = ex - 1 */
  int shared = ex - 1 - 2;
  if (shared < -127) shared = -127;
  if (shared > 127) shared = 127;
  return shared + 127;
}

/* Blocks of 32 along block_axis (0: columns, 1: rows); codes packed like
   orc_quantize's (element or row 2i in the low nibble); scales [rows][cols/32]
   or [rows/32][cols]. */
void orc_mx_quantize(const float* x, int64_t rows, int64_t cols, int block_axis, uint8_t* codes, uint8_t* scales) {
  int64_t nb = block_axis == 0 ? rows * (cols / 32) : (rows / 32) * cols;
  for (int64_t blk = 0; blk < nb; ++blk) {
    double y[32];
    int64_t idx[32];
    for (int t = 0; t < 32; ++t) {
      int64_t r, c;
      if (block_axis == 0) { r = blk / (cols / 32); c = (blk % (cols / 32)) * 32 + t; }
      else { r = (blk / cols) * 32 + t; c = blk % cols; }
      idx[t] = r * cols + c;
      y[t] = x[idx[t]];
    }
    double a = 0.0;
    int nonfinite = 0;
    for (int t = 0; t < 32; ++t) {
      if (!isfinite(y[t])) nonfinite = 1;
      else if (fabs(y[t]) > a) a = fabs(y[t]);
    }
    int sb = nonfinite ? 0xFF : orc_mx_scale_byte(a);
    double X = ldexp(1.0, sb - 127);
    scales[blk] = (uint8_t)sb;
    for (int t = 0; t < 32; ++t) {
      int code = 0;
      if (sb != 0xFF) code = orc_e2m1_encode(fabs(y[t]) / X);  /* (a zero block: every t is 0) */
      if (sb != 0xFF && signbit(y[t])) code |= 8;
      int64_t r = idx[t] / cols, c = idx[t] % cols;
      int64_t byte, shift;
      if (block_axis == 0) { byte = r * (cols / 2) + c / 2; shift = (c & 1) * 4; }
      else { byte = (r / 2) * cols + c; shift = (r & 1) * 4; }
      codes[byte] = (uint8_t)((codes[byte] & ~(0xF << shift)) | (code << shift));
    }
  }
}

void orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, int block_axis,
                       double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      int code, sb;
      if (block_axis == 0) {
        code = (codes[r * (cols / 2) + c / 2] >> ((c & 1) * 4)) & 0xF;
        sb = scales[r * (cols / 32) + c / 32];
      } else {
        code = (codes[(r / 2) * cols + c] >> ((r & 1) * 4)) & 0xF;
        sb = scales[(r / 32) * cols + c];
      }
      out[r * cols + c] = sb == 0xFF ? NAN : orc_e2m1_value(code) * ldexp(1.0, sb - 127);
    }
}

static double* mx_quant_dequant(const float* x, int64_t S, int d, int axis) {
  uint8_t* codes = (uint8_t*)calloc((size_t)(S * d / 2), 1);
  uint8_t* scales = (uint8_t*)calloc((size_t)(S * d / 32), 1);
  double* out = (double*)malloc(sizeof(double) * (size_t)(S * d));
  orc_mx_quantize(x, S, d, axis, codes, scales);
  orc_mx_dequantize(codes, scales, S, d, axis, out);
  free(codes);
  free(scales);
  return out;
}

static double* quant_dequant(const float* x, int64_t S, int d, int axis, int ss, int fmin, int fmax) {
  uint8_t* codes = (uint8_t*)calloc((size_t)(S * d / 2), 1);
  uint8_t* scales = (uint8_t*)calloc((size_t)(S * d / 16), 1);
  double* out = (double*)malloc(sizeof(double) * (size_t)(S * d));
  float g = 1.0f;
  orc_quantize(x, S, d, axis, ss, fmin, fmax, 0, &g, codes, scales, NULL);
  orc_dequantize(codes, scales, S, d, axis, 1.0f, out);
  free(codes);
  free(scales);
  return out;
}

/* Open decisions of one 16-key block of P (see attn_row): e[n] the block's
   unquantized e, P[n] its weights, V its dequantized value rows [n][d],
   amax, s2 and M the block maximum, scale byte and element factor.  Returns
   the bound in the block's own weight units (before the tile weight and the
   division by l). */
static double block_ambiguity(const float* e, const double* P, int n, const double* V, int d, float amax,
                              int s2, float M, float tm, int single_level, const double* tie) {
  double vmax[16];
  for (int j = 0; j < n; ++j) {
    vmax[j] = 0.0;
    for (int dd = 0; dd < d; ++dd)
      if (fabs(V[j * d + dd]) > vmax[j]) vmax[j] = fabs(V[j * d + dd]);
  }
  const double s2d = orc_e4m3_value(s2);
  const double lg = s2 ? log2((double)M) : 0.0;
  /* (a) codes near an E2M1 midpoint under the chosen scale */
  double codes = 0.0;
  if (s2) {
    for (int j = 0; j < n; ++j) {
      if (e[j] <= 0.0f) continue;
      const double z = log2((double)e[j]);
      const double eps = tie[0] + tie[1] * (fabs((double)tm) + fabs(lg) + fabs(z));
      const double t = (double)(e[j] * M);
      const int c0 = orc_e2m1_encode(t);
      const int lo = orc_e2m1_encode(t * (1.0 - eps)), hi = orc_e2m1_encode(t * (1.0 + eps));
      double dv = fabs(kE2M1[lo] - kE2M1[c0]);
      if (fabs(kE2M1[hi] - kE2M1[c0]) > dv) dv = fabs(kE2M1[hi] - kE2M1[c0]);
      codes += dv * s2d * vmax[j];
    }
  }
  /* (b) a neighbouring scale byte: the whole block requantized under it */
  double scale = 0.0;
  if (amax > 0.0f) {
    const double ain = single_level ? (double)(amax / 6.0f) : (double)(amax * 448.0f);
    const double eps = tie[0] + tie[1] * (fabs((double)tm) + fabs(lg) + fabs(log2((double)amax)));
    const int alts[2] = {orc_e4m3_encode(ain * (1.0 - eps)), orc_e4m3_encode(ain * (1.0 + eps))};
    for (int a = 0; a < 2; ++a) {
      const int sa = alts[a];
      if (sa == s2) continue;
      const double sad = orc_e4m3_value(sa);
      const float Ma = sa ? (single_level ? orc_recip(sa) : 2688.0f / (float)sad) : 0.0f;
      double dev = 0.0;
      for (int j = 0; j < n; ++j) {
        const double pa = sa ? kE2M1[orc_e2m1_encode((double)(e[j] * Ma))] * sad : 0.0;
        dev += fabs(pa - P[j]) * vmax[j];
      }
      if (dev > scale) scale = dev;
    }
  }
  return codes > scale ? codes : scale;
}

/* Fake-quant FP4 attention forward for one query row.
   FP4 tile (keys t0..t1-1 visible to row i):
     S_j   = Q^_i . K^_j, exact products, rounded once to binary32
     x_j   = fl32(S_j * c),  tm = max_j x_j,  e_j = exp2(fl32(x_j - tm))
     level 1 of P: the row is mapped so that e = 1 sits at 2688 = 6*448;
     level 2, per 16 consecutive keys: s2 = E4M3(fl32(amax_e * 448)) (=
       amax(2688 e)/6), elements t = fl32(e * fl32(2688 / s2)), code =
       RNE_E2M1(t), P^ = v(code) * s2 (a block with s2 = 0 is all zero)
     tile contribution: O += P^ V^ / 2688, l += sum e (unquantized, as in
       FlashAttention-2's running denominator)
   FP16 tile (a selected block pair): S_j from fp16(Q).fp16(K) rounded once
     to binary32, same x, tm, e; O += fp16(e) fp16(V), l += sum e.
   Tiles are merged with weights 2^(tm - m), m = max over tiles of tm; the
   output is O / l and lse = (m + log2 l) ln 2.  The merge order is free.

   Rounding ambiguity (tie, amb; both nullable).  The codes and block scales
   of P are integers decided by binary32 values t = e * 2688 / s2 and
   amax * 448 (single level: e / s2 and amax / 6).  An evaluation of the
   same real quantity in another order of binary32 operations (a fused
   exponent, another exp2) lands within a small relative distance of these
   values, and where a value lies that close to a rounding boundary either
   decision is a correct rounding.  With tie = {a, b}, a decision counts as
   open when moving its input by the relative slack
     eps = a + b (|tm| + |lg| + |z|),
   (z = x - tm of the element, or of the block maximum for the scale; lg =
   log2 of the element factor: 2688 / s2, or 1 / s2 single-level) changes it.
   *amb receives an upper bound on how far the row's output can move, in
   max-abs over d, when open decisions go the other way: per block, the
   larger of (a) the sum over keys with an open code of |v(alt) - v(code)|
   s2 max_c |V^_j[c]| and (b) the change of the whole block under an open
   neighbouring scale byte, weighted like the tile's output and divided by
   l (which sums the unquantized e, so it does not move).  FP16 tiles and the
   MXFP4 mode contribute nothing (their P has no such codes here, or is not
   covered). */
static void attn_row(const double* qh, const double* q16, const double* Kh, const double* Vh,
                     const double* K16, const double* V16, int64_t Sk, int d, int64_t i,
                     int causal, float c, int kv_tile, const int32_t* sel, int nsel, int sel_block,
                     int pmode, float* out, float* lse, double* Prow, double* Phrow,
                     const double* tie, double* amb) {
  /* pmode: P on the FP4 tiles -- 0 two-level NVFP4, 1 single-level NVFP4,
     2 MXFP4 (32-key blocks, power-of-two scale by the OCP rule) */
  const int single_level = pmode != 0;
  /* Prow, Phrow (nullable, Sk entries): the row's normalized probabilities,
     e * 2^(tm - m) / l, and the normalized weights the output uses, the same
     with P^ in place of e (divided by 2688 on two-level FP4 tiles); zero on
     masked keys.  Used by the training oracle. */
  int64_t ntiles = (Sk + kv_tile - 1) / kv_tile;
  float* erow = Prow ? (float*)calloc((size_t)Sk, sizeof(float)) : NULL;
  double* qrow = Prow ? (double*)calloc((size_t)Sk, sizeof(double)) : NULL;
  double* Oacc = (double*)calloc((size_t)d, sizeof(double));
  double* Ot = (double*)malloc(sizeof(double) * (size_t)d);
  float* x = (float*)malloc(sizeof(float) * (size_t)kv_tile);
  float* e = (float*)malloc(sizeof(float) * (size_t)kv_tile);
  double* P = (double*)malloc(sizeof(double) * (size_t)kv_tile);
  /* first pass: tile maxima, to know m */
  int64_t last = causal ? (i < Sk ? i : Sk - 1) : Sk - 1;
  float* tms = (float*)malloc(sizeof(float) * (size_t)ntiles);
  double* ls = (double*)malloc(sizeof(double) * (size_t)ntiles);
  double** Os = (double**)calloc((size_t)ntiles, sizeof(double*));
  int* isfp4 = (int*)malloc(sizeof(int) * (size_t)ntiles);
  double* ambs = (double*)calloc((size_t)ntiles, sizeof(double));
  float m = -INFINITY;
  int64_t T;
  for (T = 0; T < ntiles; ++T) {
    int64_t t0 = T * kv_tile, t1 = t0 + kv_tile < Sk ? t0 + kv_tile : Sk;
    if (t0 > last) break;
    if (t1 > last + 1) t1 = last + 1;
    int n = (int)(t1 - t0);
    int promoted = 0;
    for (int s = 0; s < nsel; ++s)
      if (sel[s] == (int32_t)(t0 / sel_block)) promoted = 1;
    const double* qq = promoted ? q16 : qh;
    const double* KK = promoted ? K16 : Kh;
    float tm = -INFINITY;
    for (int j = 0; j < n; ++j) {
      double s = 0.0;
      for (int dd = 0; dd < d; ++dd) s += qq[dd] * KK[(t0 + j) * d + dd];
      float S = (float)s;
      x[j] = S * c;
      if (x[j] > tm) tm = x[j];
    }
    /* MXFP4 tiles take the power of two at or above the tile maximum as their
       reference (the row level of P can only be a power of two with E8M0
       block scales): e = 2^(x - ceil(tm)) in (1/2, 1] at the maximum */
    if (pmode == 2 && !promoted) tm = ceilf(tm);
    double lsum = 0.0;
    for (int j = 0; j < n; ++j) {
      float z = x[j] - tm;
      e[j] = exp2_f32(z);
      lsum += (double)e[j];
    }
    if (promoted) {
      for (int j = 0; j < n; ++j) P[j] = orc_round_fp16((double)e[j]);
    } else if (pmode == 2) {
      for (int b0 = 0; b0 < n; b0 += 32) {
        int b1 = b0 + 32 < n ? b0 + 32 : n;
        float amax = 0.0f;
        for (int j = b0; j < b1; ++j)
          if (e[j] > amax) amax = e[j];
        int sb = orc_mx_scale_byte((double)amax);
        double X = ldexp(1.0, sb - 127);
        for (int j = b0; j < b1; ++j) P[j] = kE2M1[orc_e2m1_encode((double)e[j] / X)] * X;
      }
    } else {
      for (int b0 = 0; b0 < n; b0 += 16) {
        int b1 = b0 + 16 < n ? b0 + 16 : n;
        float amax = 0.0f;
        for (int j = b0; j < b1; ++j)
          if (e[j] > amax) amax = e[j];
        /* two-level: the row level maps e = 1 to 2688, so the block scale is
           E4M3(amax * 2688 / 6) = E4M3(amax * 448) and the element factor
           fl32(2688 / s2); single level (Attn-QAT page, Metodologia / B: no
           two-level step): the block scale is E4M3(fl32(amax / 6)) and the
           element factor the correctly rounded reciprocal R(s2), as in the
           quantizer */
        int s2 = single_level ? orc_e4m3_encode((double)(amax / 6.0f)) : orc_e4m3_encode((double)(amax * 448.0f));
        if (s2 == 0) {
          for (int j = b0; j < b1; ++j) P[j] = 0.0;
          continue;
        }
        float s2f = (float)orc_e4m3_value(s2);
        float M = single_level ? orc_recip(s2) : 2688.0f / s2f;
        for (int j = b0; j < b1; ++j) {
          float t = e[j] * M;
          int code = orc_e2m1_encode((double)t);
          P[j] = kE2M1[code] * (double)s2f;
        }
        if (tie) ambs[T] += block_ambiguity(e + b0, P + b0, b1 - b0, Vh + (t0 + b0) * d, d, amax, s2, M,
                                            tm, single_level, tie);
      }
    }
    const double* VV = promoted ? V16 : Vh;
    double* O = (double*)calloc((size_t)d, sizeof(double));
    for (int j = 0; j < n; ++j)
      if (P[j] != 0.0)
        for (int dd = 0; dd < d; ++dd) O[dd] += P[j] * VV[(t0 + j) * d + dd];
    if (!promoted && !single_level)
      for (int dd = 0; dd < d; ++dd) O[dd] /= 2688.0;
    if (erow)
      for (int j = 0; j < n; ++j) {
        erow[t0 + j] = e[j];
        qrow[t0 + j] = (!promoted && !single_level) ? P[j] / 2688.0 : P[j];
      }
    Os[T] = O;
    tms[T] = tm;
    ls[T] = lsum;
    isfp4[T] = !promoted;
    if (tm > m) m = tm;
  }
  int64_t nt = T;
  double l = 0.0, am = 0.0;
  for (T = 0; T < nt; ++T) {
    double r = exp2((double)tms[T] - (double)m);
    l += r * ls[T];
    am += r * ambs[T];
    for (int dd = 0; dd < d; ++dd) Oacc[dd] += r * Os[T][dd];
    free(Os[T]);
  }
  if (amb) *amb = nt ? am / (single_level ? 1.0 : 2688.0) / l : 0.0;
  for (int dd = 0; dd < d; ++dd) out[dd] = nt ? (float)(Oacc[dd] / l) : 0.0f;
  if (lse) *lse = nt ? (float)(((double)m + log2(l)) * 0.69314718055994530942) : -INFINITY;
  if (Prow) {
    for (int64_t j = 0; j < Sk; ++j) { Prow[j] = 0.0; Phrow[j] = 0.0; }
    for (T = 0; T < nt; ++T) {
      double r = exp2((double)tms[T] - (double)m);
      int64_t t0 = T * kv_tile, t1 = t0 + kv_tile < Sk ? t0 + kv_tile : Sk;
      if (t1 > last + 1) t1 = last + 1;
      for (int64_t j = t0; j < t1; ++j) {
        Prow[j] = (double)erow[j] * r / l;
        Phrow[j] = qrow[j] * r / l;
      }
    }
    free(erow); free(qrow);
  }
  (void)isfp4;
  free(isfp4); free(ambs); free(Os); free(ls); free(tms); free(P); free(e); free(x); free(Ot); free(Oacc);
}

/* Forward FP4 attention over q [B][H][Sq][d], k and v [B][Hkv][Sk][d]
   (binary32 copies of the bf16/fp16 inputs).  Q and K are quantized in blocks
   along d, V in blocks of 16 tokens (each block runs along the reduction axis
   of its product), with ScaleSearch per the arguments and no per-tensor scale.
   pct > 0 enables block selection with sel_block-token blocks.
   rows (n_rows of them, NULL = all) picks the query rows; heads (n_heads, NULL
   = all) picks flattened b*H+h heads.  out is [n_heads][n_rows][d], lse
   [n_heads][n_rows] (nullable); topk_idx [n_heads][nqb][kmax] and topk_cnt
   [n_heads][nqb] (nullable) receive the selection.  single_level quantizes P
   with the NVFP4 block scale alone (no row level; the Attn-QAT page removes
   the two-level step).  probs and probs_hat (nullable, both or neither,
   [n_heads][n_rows][Sk]) receive every row's normalized probabilities and the
   normalized weights the output uses (see attn_row).  tie (nullable, {a, b})
   and amb (nullable, [n_heads][n_rows]) give every row's rounding-ambiguity
   bound (see attn_row).  Returns 0, or -1 on bad arguments. */
int orc_attention_fwd(const float* q, const float* k, const float* v, int B, int H, int Hkv,
                      int64_t Sq, int64_t Sk, int d, int causal, double softmax_scale, int kv_tile,
                      int scale_search, int fmin, int fmax, int pct, int sel_block,
                      const int64_t* rows, int64_t n_rows, const int* heads, int n_heads,
                      float* out, float* lse, int32_t* topk_idx, int32_t* topk_cnt,
                      const float* q_fp4, const float* k_fp4, int single_level,
                      double* probs, double* probs_hat, int mx, const double* tie, double* amb) {
  /* mx: Q, K (blocks of 32 along d), V (blocks of 32 tokens) and P (blocks of
     32 keys) in MXFP4 instead of NVFP4 (scale_search does not apply) */
  const int pmode = mx ? 2 : (single_level ? 1 : 0);
  if (mx && (d % 32 || Sk % 32 || kv_tile % 32)) return -1;
  /* q_fp4, k_fp4 (nullable, same layout as q, k): what the FP4 path
     quantizes, e.g. Q and K after incoherence processing; the FP16 path and
     the block means always use q and k. */
  if (!q_fp4) q_fp4 = q;
  if (!k_fp4) k_fp4 = k;
  if (d % 16 || Sk % 16 || kv_tile % 16 || H % Hkv) return -1;
  if (causal && Sq != Sk) return -1;
  if (pct > 0 && sel_block % kv_tile) return -1;
  float c = orc_score_factor(softmax_scale, d);
  int nh = heads ? n_heads : B * H;
  int64_t nr = rows ? n_rows : Sq;
  int nqb = (int)((Sq + sel_block - 1) / sel_block), nkb = (int)((Sk + sel_block - 1) / sel_block);
  int kmax = pct > 0 ? orc_topk_count(pct, nkb) : 0;
  for (int hi = 0; hi < nh; ++hi) {
    int bh = heads ? heads[hi] : hi;
    int b = bh / H, h = bh % H, hk = h / (H / Hkv);
    const float* qb = q + ((int64_t)b * H + h) * Sq * d;
    const float* kb = k + ((int64_t)b * Hkv + hk) * Sk * d;
    const float* vb = v + ((int64_t)b * Hkv + hk) * Sk * d;
    const float* qbr = q_fp4 + ((int64_t)b * H + h) * Sq * d;
    const float* kbr = k_fp4 + ((int64_t)b * Hkv + hk) * Sk * d;
    double* Kh = mx ? mx_quant_dequant(kbr, Sk, d, 0) : quant_dequant(kbr, Sk, d, 0, scale_search, fmin, fmax);
    double* Vh = mx ? mx_quant_dequant(vb, Sk, d, 1) : quant_dequant(vb, Sk, d, 1, scale_search, fmin, fmax);
    double* Qmx = mx ? mx_quant_dequant(qbr, Sq, d, 0) : NULL;
    double *K16 = NULL, *V16 = NULL;
    int32_t* sidx = NULL;
    int32_t* scnt = NULL;
    if (pct > 0) {
      K16 = (double*)malloc(sizeof(double) * (size_t)(Sk * d));
      V16 = (double*)malloc(sizeof(double) * (size_t)(Sk * d));
      for (int64_t t = 0; t < Sk * d; ++t) { K16[t] = orc_round_fp16(kb[t]); V16[t] = orc_round_fp16(vb[t]); }
      double* qm = (double*)malloc(sizeof(double) * (size_t)nqb * d);
      double* km = (double*)malloc(sizeof(double) * (size_t)nkb * d);
      orc_block_means(qb, Sq, d, sel_block, qm);
      orc_block_means(kb, Sk, d, sel_block, km);
      sidx = (int32_t*)malloc(sizeof(int32_t) * (size_t)nqb * kmax);
      scnt = (int32_t*)malloc(sizeof(int32_t) * (size_t)nqb);
      orc_block_topk(qm, km, nqb, nkb, d, causal, pct, kmax, sidx, scnt);
      if (topk_idx) memcpy(topk_idx + (int64_t)hi * nqb * kmax, sidx, sizeof(int32_t) * (size_t)nqb * kmax);
      if (topk_cnt) memcpy(topk_cnt + (int64_t)hi * nqb, scnt, sizeof(int32_t) * (size_t)nqb);
      free(qm); free(km);
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nr; ++ri) {
      int64_t i = rows ? rows[ri] : ri;
      /* Q row quantized on its own: its blocks lie inside the row */
      uint8_t cd[16], sc;
      int8_t of;
      double* qh = (double*)malloc(sizeof(double) * (size_t)d);
      double* q16 = (double*)malloc(sizeof(double) * (size_t)d);
      if (mx) {
        for (int dd = 0; dd < d; ++dd) qh[dd] = Qmx[i * d + dd];
      } else {
        for (int blk = 0; blk < d / 16; ++blk) {
          orc_quantize_block(qbr + i * d + blk * 16, 1, scale_search, fmin, fmax, cd, &sc, &of, NULL);
          for (int t = 0; t < 16; ++t) qh[blk * 16 + t] = orc_e2m1_value(cd[t]) * orc_e4m3_value(sc);
        }
      }
      for (int dd = 0; dd < d; ++dd) q16[dd] = orc_round_fp16(qb[i * d + dd]);
      const int32_t* sel = NULL;
      int nsel = 0;
      if (pct > 0) {
        int qbk = (int)(i / sel_block);
        sel = sidx + (int64_t)qbk * kmax;
        nsel = scnt[qbk];
      }
      attn_row(qh, q16, Kh, Vh, K16, V16, Sk, d, i, causal, c, kv_tile, sel, nsel, sel_block, pmode,
               out + ((int64_t)hi * nr + ri) * d, lse ? lse + (int64_t)hi * nr + ri : NULL,
               probs ? probs + ((int64_t)hi * nr + ri) * Sk : NULL,
               probs ? probs_hat + ((int64_t)hi * nr + ri) * Sk : NULL,
               amb ? tie : NULL, amb ? amb + (int64_t)hi * nr + ri : NULL);
      free(qh); free(q16);
    }
    free(Kh); free(Vh); free(Qmx); free(K16); free(V16); free(sidx); free(scnt);
  }
  return 0;
}

/* Plain softmax attention in binary64: out = softmax(scale * q k^T) v with the
   top-left causal mask (key j visible to query i iff j <= i).  Same argument
   conventions as orc_attention_fwd (rows/heads selection). */
int orc_attention_exact(const float* q, const float* k, const float* v, int B, int H, int Hkv,
                        int64_t Sq, int64_t Sk, int d, int causal, double softmax_scale,
                        const int64_t* rows, int64_t n_rows, const int* heads, int n_heads,
                        float* out, float* lse) {
  if (H % Hkv) return -1;
  double sc = softmax_scale > 0.0 ? softmax_scale : 1.0 / sqrt((double)d);
  int nh = heads ? n_heads : B * H;
  int64_t nr = rows ? n_rows : Sq;
  for (int hi = 0; hi < nh; ++hi) {
    int bh = heads ? heads[hi] : hi;
    int b = bh / H, h = bh % H, hk = h / (H / Hkv);
    const float* qb = q + ((int64_t)b * H + h) * Sq * d;
    const float* kb = k + ((int64_t)b * Hkv + hk) * Sk * d;
    const float* vb = v + ((int64_t)b * Hkv + hk) * Sk * d;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t ri = 0; ri < nr; ++ri) {
      int64_t i = rows ? rows[ri] : ri;
      int64_t n = causal ? (i + 1 < Sk ? i + 1 : Sk) : Sk;
      double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
      double mx = -INFINITY;
      for (int64_t j = 0; j < n; ++j) {
        double a = 0.0;
        for (int dd = 0; dd < d; ++dd) a += (double)qb[i * d + dd] * (double)kb[j * d + dd];
        s[j] = a * sc;
        if (s[j] > mx) mx = s[j];
      }
      double l = 0.0;
      for (int64_t j = 0; j < n; ++j) { s[j] = exp(s[j] - mx); l += s[j]; }
      float* o = out + ((int64_t)hi * nr + ri) * d;
      for (int dd = 0; dd < d; ++dd) {
        double a = 0.0;
        for (int64_t j = 0; j < n; ++j) a += s[j] * (double)vb[j * d + dd];
        o[dd] = n ? (float)(a / l) : 0.0f;
      }
      if (lse) lse[(int64_t)hi * nr + ri] = n ? (float)(mx + log(l)) : -INFINITY;
      free(s);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Decode over a sink-aware mixed-precision KV cache                         */
/* ([ScaleSearch] Metodologia / ScaleSearchAttention, cache paragraph)       */
/* ------------------------------------------------------------------------ */

/* One query token per (batch, q-head) against a context of L_b = ctx_len[b]
   tokens.  Reading: the first n_sink and the last n_recent tokens stay in
   bf16; the middle M_b = L_b - n_sink - n_recent tokens (a multiple of 16) are
   stored NVFP4: K in blocks along d, V in blocks of 16 tokens starting at the
   first middle token, both quantized with ScaleSearch per the arguments and no
   per-tensor scale.  q stays unquantized.  The output is the plain binary64
   softmax attention over that dequantized cache.
   q [B][Hq][d]; k, v [B][Hkv][Lcap][d] hold the original context.
   pairs (n_pairs of them, NULL = all) picks flattened b*Hkv+kvh pairs; out is
   [n_pairs][Hq/Hkv][d], lse [n_pairs][Hq/Hkv] (natural log).
   With pct > 0 (ThriftAttention page, Metodologia / 1 and / 2, applied to
   decode; reading: the query block of a kv head is its G query tokens, and the
   cache keeps a full-precision copy of the middle beside the NVFP4 one), the
   middle is cut into blocks of sel_blk tokens from its first token (the last
   one may be short), each block j is scored by mean(q over the G heads) .
   mean(K block j) in binary64 (orc_block_means / orc_block_topk order), and
   the ceil(pct * n / 100) best blocks take their original K and V instead of
   the dequantized ones.  sel_idx [n_pairs][kmax] (ascending, -1 padded) and
   sel_cnt [n_pairs] (nullable) receive the choice.  Returns 0, or -1 on bad
   arguments. */
int orc_attention_decode(const float* q, const float* k, const float* v, const int32_t* ctx_len,
                         int B, int Hq, int Hkv, int d, int64_t Lcap, int n_sink, int n_recent,
                         double softmax_scale, int scale_search, int fmin, int fmax,
                         const int* pairs, int n_pairs, float* out, float* lse,
                         int pct, int sel_blk, int kmax, int32_t* sel_idx, int32_t* sel_cnt) {
  if (Hq % Hkv || d % 16) return -1;
  if (pct < 0 || pct > 100 || (pct > 0 && sel_blk < 1)) return -1;
  int G = Hq / Hkv;
  double sc = softmax_scale > 0.0 ? softmax_scale : 1.0 / sqrt((double)d);
  int np = pairs ? n_pairs : B * Hkv;
  for (int pi = 0; pi < np; ++pi) {
    int bk = pairs ? pairs[pi] : pi;
    int b = bk / Hkv, hk = bk % Hkv;
    int64_t L = ctx_len[b];
    int64_t M = L - n_sink - n_recent;
    if (L > Lcap || M < 0 || M % 16) return -1;
    const float* kb = k + ((int64_t)b * Hkv + hk) * Lcap * d;
    const float* vb = v + ((int64_t)b * Hkv + hk) * Lcap * d;
    double* Kt = (double*)malloc(sizeof(double) * (size_t)(L * d));
    double* Vt = (double*)malloc(sizeof(double) * (size_t)(L * d));
    for (int64_t t = 0; t < L * d; ++t) { Kt[t] = kb[t]; Vt[t] = vb[t]; }
    if (M > 0) {
      double* Kq = quant_dequant(kb + (int64_t)n_sink * d, M, d, 0, scale_search, fmin, fmax);
      double* Vq = quant_dequant(vb + (int64_t)n_sink * d, M, d, 1, scale_search, fmin, fmax);
      memcpy(Kt + (int64_t)n_sink * d, Kq, sizeof(double) * (size_t)(M * d));
      memcpy(Vt + (int64_t)n_sink * d, Vq, sizeof(double) * (size_t)(M * d));
      free(Kq); free(Vq);
    }
    /* Selective promotion: the middle's key blocks of sel_blk tokens are
       scored against the mean of the group's G query vectors and the best
       ceil(pct * n / 100) are read from the full-precision copy. */
    if (pct > 0) {
      int nb = (int)((M + sel_blk - 1) / sel_blk);
      int k_b = orc_topk_count(pct, nb);
      if (k_b > kmax) { free(Kt); free(Vt); return -1; }
      int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(kmax > 0 ? kmax : 1));
      int32_t cnt = 0;
      for (int w = 0; w < kmax; ++w) idx[w] = -1;
      if (nb > 0) {
        double* km = (double*)malloc(sizeof(double) * (size_t)nb * d);
        double* qm = (double*)malloc(sizeof(double) * (size_t)d);
        orc_block_means(kb + (int64_t)n_sink * d, M, d, sel_blk, km);
        for (int dd = 0; dd < d; ++dd) {
          double s = 0.0;
          for (int g = 0; g < G; ++g) s += (double)q[((int64_t)b * Hq + hk * G + g) * d + dd];
          qm[dd] = s / (double)G;
        }
        orc_block_topk(qm, km, 1, nb, d, 0, pct, kmax > 0 ? kmax : 1, idx, &cnt);
        for (int w = 0; w < cnt; ++w) {
          int64_t t0 = n_sink + (int64_t)idx[w] * sel_blk;
          int64_t t1 = t0 + sel_blk < n_sink + M ? t0 + sel_blk : n_sink + M;
          for (int64_t t = t0 * d; t < t1 * d; ++t) { Kt[t] = kb[t]; Vt[t] = vb[t]; }
        }
        free(km); free(qm);
      }
      if (sel_idx) memcpy(sel_idx + (int64_t)pi * kmax, idx, sizeof(int32_t) * (size_t)kmax);
      if (sel_cnt) sel_cnt[pi] = cnt;
      free(idx);
    }
#pragma omp parallel for schedule(static)
    for (int g = 0; g < G; ++g) {
      int h = hk * G + g;
      const float* qq = q + ((int64_t)b * Hq + h) * d;
      double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
      double mx = -INFINITY;
      for (int64_t j = 0; j < L; ++j) {
        double a = 0.0;
        for (int dd = 0; dd < d; ++dd) a += (double)qq[dd] * Kt[j * d + dd];
        s[j] = a * sc;
        if (s[j] > mx) mx = s[j];
      }
      double l = 0.0;
      for (int64_t j = 0; j < L; ++j) { s[j] = exp(s[j] - mx); l += s[j]; }
      float* o = out + ((int64_t)pi * G + g) * d;
      for (int dd = 0; dd < d; ++dd) {
        double a = 0.0;
        for (int64_t j = 0; j < L; ++j) a += s[j] * Vt[j * d + dd];
        o[dd] = L ? (float)(a / l) : 0.0f;
      }
      if (lse) lse[(int64_t)pi * G + g] = L ? (float)(mx + log(l)) : -INFINITY;
      free(s);
    }
    free(Kt); free(Vt);
  }
  return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

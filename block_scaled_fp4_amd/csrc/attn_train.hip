// attn_train.hip -- backward of FP4 attention for quantization-aware training
// (Attn-QAT page, Metodologia / A: the probabilities are recomputed in FP4 in
// the backward, as the forward used them; the row term of the softmax
// gradient uses the high-precision output O' kept by the forward).
//
// With fake-quantized operands Q^, K^, V^ (NVFP4, straight-through), the
// normalized probabilities P = 2^(x - lse2) (x = fl32(S c), S = Q^ K^T) and the
// normalized FP4 weights P^ the forward's output used (tile-local
// quantization of e = 2^(x - tm), rescaled by 2^(tm - lse2)):
//   dV = P^T dO,  dS = s P * (dO V^T - D),  D = rowsum(dO * O'),
//   dQ = dS K^,   dK = dS^T Q^,             s = c ln 2.
// Nothing score-sized is stored: one kernel per key tile recomputes the
// scores, P, P^ and dS for every query that sees the tile and accumulates dK
// and dV (summed over the query heads of a kv head); one kernel per query
// tile recomputes the scores, P and dS and accumulates dQ.  The products run
// on the bf16 MFMA with binary32 accuracy; the workspace holds bf16 copies of
// the operands (exact) and D only.
#include "device_common.h"
#include "fp4_internal.h"

namespace fp4dev {

constexpr int kGT = 128;  // query rows per dQ workgroup, keys per dK/dV workgroup

// ---- operands in bf16 -------------------------------------------------------
//
// The dequantized NVFP4 operands are bf16 numbers (an E2M1 value times an
// E4M3 scale has at most 6 significant bits, within bf16's exponent range),
// so their bf16 copies are exact: the top half of the binary32 pattern.

__device__ __forceinline__ uint32_t bf16x2_exact(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

// NVFP4 rows with blocks along the row (Q, K): codes [rows, d/2], scales
// [rows, d/16] -> bf16 [rows, d].  One thread per 8 codes (4 bytes).
__global__ void __launch_bounds__(256) dequant_rows_kernel(const uint8_t* codes, const uint8_t* scales,
                                                           int64_t rows, int d, uint16_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // group of 8 elements
  const int64_t n = rows * (d / 8);
  if (i >= n) return;
  const int64_t r = i / (d / 8);
  const int c8 = (int)(i % (d / 8));
  const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + r * (d / 2) + 4 * c8);
  const float s = e4m3_to_f32(scales[r * (d / 16) + c8 / 2]);
  const float2_t v0 = cvt_pk_f32_fp4<0>(w), v1 = cvt_pk_f32_fp4<1>(w);
  const float2_t v2 = cvt_pk_f32_fp4<2>(w), v3 = cvt_pk_f32_fp4<3>(w);
  *reinterpret_cast<uint4_t*>(out + r * d + 8 * c8) =
      uint4_t{bf16x2_exact(v0[0] * s, v0[1] * s), bf16x2_exact(v1[0] * s, v1[1] * s),
              bf16x2_exact(v2[0] * s, v2[1] * s), bf16x2_exact(v3[0] * s, v3[1] * s)};
}

// NVFP4 with blocks of 16 rows (V): codes [rows/2, d] (row 2i in the low
// nibble), scales [rows/16, d] -> bf16 [rows, d].  One thread per row pair
// and column.
__global__ void __launch_bounds__(256) dequant_cols_kernel(const uint8_t* codes, const uint8_t* scales,
                                                           int64_t rows, int d, uint16_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (rows / 2) * d;
  if (i >= n) return;
  const int64_t pr = i / d;
  const int c = (int)(i % d);
  const uint32_t b = codes[pr * d + c];
  const float s = e4m3_to_f32(scales[(pr / 8) * d + c]);
  const float2_t v = cvt_pk_f32_fp4<0>(b);
  const uint32_t pk = bf16x2_exact(v[0] * s, v[1] * s);
  out[(2 * pr) * d + c] = (uint16_t)pk;
  out[(2 * pr + 1) * d + c] = (uint16_t)(pk >> 16);
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }
template <>
__device__ __forceinline__ float to_f32<half_t>(half_t v) { return (float)v; }
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // finite values only
}

// fp16 dO is not a bf16 number: x = hi + lo exactly with hi = bf16(x), lo = bf16(x - hi)
// (11 significant bits fit in two bf16 terms of 8)
__global__ void __launch_bounds__(256) split_f16_kernel(const half_t* x, int64_t n, uint16_t* hi, uint16_t* lo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = (float)x[i];
  const uint32_t h = bf16_rne_bits(v);
  hi[i] = (uint16_t)h;
  lo[i] = (uint16_t)bf16_rne_bits(v - __uint_as_float(h << 16));
}

// 8 consecutive elements (16-byte aligned) as binary32
template <typename T>
__device__ __forceinline__ void load8f(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8f<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const uint4_t w = *reinterpret_cast<const uint4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void load8f<half_t>(const half_t* p, float (&v)[8]) {
  const half8_t w = *reinterpret_cast<const half8_t*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)w[i];
}
template <>
__device__ __forceinline__ void load8f<float>(const float* p, float (&v)[8]) {
  const float4_t a = *reinterpret_cast<const float4_t*>(p), b = *reinterpret_cast<const float4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

// D[row] = sum_d dO[row][d] O'[row][d] in binary32: 16 lanes per row, each
// with 8 consecutive elements (16-byte loads), then a sum over the 16 lanes.
template <typename TD, typename TO>
__global__ void __launch_bounds__(256) row_dot_kernel(const TD* dout, const TO* ohp, int64_t rows, int d, float* D) {
  const int sub = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  float s = 0.0f;
  if (row < rows) {
    for (int c = 8 * sub; c < d; c += 128) {
      float a[8], b[8];
      load8f<TD>(dout + row * d + c, a);
      load8f<TO>(ohp + row * d + c, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) s = __builtin_fmaf(a[e], b[e], s);
    }
  }
#pragma unroll
  for (int k = 8; k > 0; k >>= 1) s += __shfl_xor(s, k, 64);  // within the row's 16 lanes
  if (sub == 0 && row < rows) D[row] = s;
}

// ---- probabilities --------------------------------------------------------

// Per E4M3 byte of the P block scale: {factor, s2} with factor the element
// multiplier of the quantization input (two-level: fl32(2688 / s2); single
// level: the correctly rounded 1 / s2), as the forward's definition.
struct TrainPTable {
  float2_t two[128];
  float2_t one[128];
  constexpr TrainPTable() : two(), one() {
    for (int b = 0; b < 128; ++b) {
      double s2 = 0.0;
      if (b < 8) s2 = (double)b / 512.0;
      else {
        int e = (b >> 3) - 7, mm = b & 7;
        s2 = 1.0 + (double)mm / 8.0;
        for (int i = 0; i < e; ++i) s2 *= 2.0;
        for (int i = 0; i > e; --i) s2 /= 2.0;
      }
      const bool ok = b != 0 && b != 127;
      two[b] = ok ? float2_t{(float)(2688.0 / s2), (float)s2} : float2_t{0.0f, 0.0f};
      one[b] = ok ? float2_t{(float)(1.0 / s2), (float)s2} : float2_t{0.0f, 0.0f};
    }
  }
};
__constant__ TrainPTable kTrainP = TrainPTable();

// ---- binary32 products on the bf16 MFMA --------------------------------------
//
// The products keep binary32 accuracy on the bf16 matrix instructions: an
// operand whose values are bf16 numbers (the dequantized NVFP4 Q^, K^, V^ --
// an E2M1 value times an E4M3 scale has at most 6 significant bits -- and dO
// given in bf16) goes in as it is; an fp32 operand (P^, dS) is split as
// x = hi + lo + r with |r| <= 2^-16 |x| (see pack8), and an fp16 dO exactly
// as hi + lo; each product takes hi.B + lo.B (with an fp16 dO on the other
// side, hi.lo too; the dropped lo.lo term is below 2^-14 of the product).
// Products are exact in the MFMA and accumulate in fp32.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// 4 fp32 -> 4 bf16 hi (and lo when SPLIT), packed two per dword
template <bool SPLIT>
__device__ __forceinline__ void split4(const float4_t& x, uint2_t& hi, uint2_t& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = bf16_rne_bits(x[i]);
    l[i] = SPLIT ? bf16_rne_bits(x[i] - __uint_as_float(h[i] << 16)) : 0u;  // the difference is exact
  }
  hi = uint2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  lo = uint2_t{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
}

__device__ __forceinline__ float16_t mfma_bf16(const uint4_t& a, const uint4_t& b, const float16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// 8 consecutive bf16 of a row as one MFMA operand (zero when !ok)
__device__ __forceinline__ uint4_t fragb(const uint16_t* p, bool ok) {
  return ok ? *reinterpret_cast<const uint4_t*>(p) : uint4_t{0, 0, 0, 0};
}

// 4 x 4 transpose of 16-bit elements: in[i] holds elements (i, 0..3), out[j] elements (0..3, j)
__device__ __forceinline__ void transpose4x4_16(const uint2_t (&in)[4], uint2_t (&out)[4]) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {  // columns 2w and 2w+1
    const uint32_t a = in[0][w], b = in[1][w], c = in[2][w], d = in[3][w];
    out[2 * w] = uint2_t{__builtin_amdgcn_perm(b, a, 0x05040100u), __builtin_amdgcn_perm(d, c, 0x05040100u)};
    out[2 * w + 1] = uint2_t{__builtin_amdgcn_perm(b, a, 0x07060302u), __builtin_amdgcn_perm(d, c, 0x07060302u)};
  }
}

// ---- dK and dV without materialized scores ---------------------------------
//
// One workgroup per 128-key tile of a kv head (4 waves x 32 keys), looping
// over 32-query blocks of the G query heads that read it, in two passes that
// each fit two waves per SIMD: the dV pass needs P^ (block and tile maxima),
// the dK pass needs P and dP.  The wave keeps its keys' K^ (and V^) as B
// operands in registers and recomputes S = Q^ K^T (and dP = dO V^T) with Q
// and dO rows fed in the order krow2 (bits 2 and 3 of the row swapped), which
// leaves lane (key, h) holding queries 8h..8h+7 and 16+8h..16+8h+7: exactly
// the k order of the A operand of dV += P^T dO and dK += dS^T Q^.  P^ is
// quantized as in the forward: the 16-key block maximum is a reduction over
// one 16-lane DPP row, the tile maximum over kv_tile keys goes through LDS
// across waves.

struct KvArgs {
  const uint16_t *q, *k, *v, *doh, *dol;  // bf16 [rows][d]; dol: the low terms of an fp16 dO
  const float *D, *lse;
  float *dk, *dv;
  int64_t H, G, Sq, Sk;
  int kv_tile, causal, single, nkt;
  float c, alpha;
};

__device__ __forceinline__ int krow2(int r) { return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1); }

// dV pass: K rows fed to S^T = K^ Q^T in this order leave lane (query, h)
// holding keys 16h .. 16h+15 of the wave, consecutive (the output rows of a
// 32x32 MFMA lane are 4h + 8j + i, i < 4, j < 4)
__device__ __forceinline__ int krow16(int r) { return (r & 3) | ((r >> 3) << 2) | (((r >> 2) & 1) << 4); }

__device__ __forceinline__ float max16v(const float (&a)[16]) {
  float m0 = __builtin_fmaxf(__builtin_fmaxf(a[0], a[1]), a[2]);
  float m1 = __builtin_fmaxf(__builtin_fmaxf(a[3], a[4]), a[5]);
  float m2 = __builtin_fmaxf(__builtin_fmaxf(a[6], a[7]), a[8]);
  float m3 = __builtin_fmaxf(__builtin_fmaxf(a[9], a[10]), a[11]);
  float m4 = __builtin_fmaxf(__builtin_fmaxf(a[12], a[13]), a[14]);
  m0 = __builtin_fmaxf(__builtin_fmaxf(m0, m1), m2);
  m3 = __builtin_fmaxf(__builtin_fmaxf(m3, m4), a[15]);
  return __builtin_fmaxf(m0, m3);
}

// Two binary32 values -> two bf16 (round to nearest even) in one dword, low
// half first: gfx950's packed convert.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{a, b}, bf16x2_v));
}

// 8 fp32 -> 8 bf16 (hi, and lo when SPLIT) as one MFMA operand.  Without the
// split the values are bf16 numbers and hi is exact.  With it, hi is x cut to
// its top 16 bits (exact difference x - hi, below 2^-7 |x|) and lo that
// difference rounded to bf16, so |x - hi - lo| <= 2^-16 |x|.
template <bool SPLIT>
__device__ __forceinline__ void pack8(const float* x, uint4_t& hi, uint4_t& lo) {
  if (!SPLIT) {
    uint2_t ha, la, hb, lb;
    split4<false>(float4_t{x[0], x[1], x[2], x[3]}, ha, la);
    split4<false>(float4_t{x[4], x[5], x[6], x[7]}, hb, lb);
    hi = uint4_t{ha[0], ha[1], hb[0], hb[1]};
    lo = uint4_t{0u, 0u, 0u, 0u};
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t a = __float_as_uint(x[2 * j]), b = __float_as_uint(x[2 * j + 1]);
    hi[j] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // top halves of a (low) and b (high)
    lo[j] = bf16x2_rne(x[2 * j] - __uint_as_float(a & 0xFFFF0000u), x[2 * j + 1] - __uint_as_float(b & 0xFFFF0000u));
  }
}

template <int D, bool SPLIT_DO, int MODE>  // MODE 0: dV, 1: dK
__global__ void __launch_bounds__(256, 2) bwd_kv_kernel(KvArgs A) {
  constexpr bool DV = MODE == 0;
  constexpr bool SPL = SPLIT_DO;
  constexpr int QB = 32;        // queries per step
  constexpr int RA = D + 8;     // [query][d] rows, bf16
  constexpr int RB = QB + 8;    // [d][query] rows, bf16
  // dV: Q^ as [query][d] (scores), dO as [d][query] (product B operand);
  // dK: Q^ in both layouts, dO as [query][d] (dP)
  __shared__ uint16_t Qa[QB * RA], Xb[D * RB];
  __shared__ uint16_t Oa[DV ? 1 : QB * RA], Oal[!DV && SPL ? QB * RA : 1], Xbl[DV && SPL ? D * RB : 1];
  __shared__ __align__(16) float lse_s[QB];
  __shared__ __align__(16) float D_s[QB];
  __shared__ __align__(16) float tmx[DV ? 8 : 1][QB];  // block maxima: [2 wave + row of the wave][query]
  __shared__ float2_t ptab[DV ? 128 : 1];             // the P-scale table of the chosen scheme
  // dV: P^ of the wave's 32 keys x the step's 32 queries as bf16 hi and lo
  // terms, [query][key] rows (padded to 40), written by (query, key half)
  // lanes and read back by (key, query half) lanes
  constexpr int RPT = 40;
  __shared__ __align__(16) uint16_t pth[DV ? 4 * QB * RPT : 1], ptl[DV ? 4 * QB * RPT : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hi = lane >> 5, r32 = lane & 31;
  const int64_t BHkv = gridDim.x / A.nkt;
  const int64_t bhk = blockIdx.x % BHkv;
  const int kt = (int)(blockIdx.x / BHkv);  // key tile 0 sees the most queries under the causal mask
  const int64_t Hkv = A.H / A.G;
  const int64_t b = bhk / Hkv, hk = bhk - b * Hkv;
  const int64_t key0 = (int64_t)kt * kGT;
  const int64_t key = key0 + 32 * wave + r32;
  const bool kok = key < A.Sk;
  // the K^ row this lane feeds: key r32 (dK: B operand), key krow16(r32) (dV: A operand of S^T)
  const int64_t kfeed = key0 + 32 * wave + (DV ? krow16(r32) : r32);
  const bool fok = kfeed < A.Sk;
  uint4_t kf[D / 16], vf[DV ? 1 : D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kf[s] = fragb(A.k + (bhk * A.Sk + (fok ? kfeed : 0)) * D + 16 * s + 8 * hi, fok);
    if (!DV) vf[DV ? 0 : s] = fragb(A.v + (bhk * A.Sk + (kok ? key : 0)) * D + 16 * s + 8 * hi, kok);
  }
  float16_t acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc[t] = float16_t{0};
  if (DV && threadIdx.x < 128) ptab[threadIdx.x] = A.single ? kTrainP.one[threadIdx.x] : kTrainP.two[threadIdx.x];
  const int64_t qstart = A.causal ? key0 : 0;  // earlier queries see none of these keys
  const int nqb = qstart < A.Sq ? (int)((A.Sq - qstart + QB - 1) / QB) : 0;
  const int nsteps = (int)A.G * nqb;  // (query head, query block) pairs
  const int qr = krow2(r32);  // the Q / dO row this lane feeds to the score products
  auto qof = [&](int v) { return (v & 7) + 8 * hi + 16 * (v >> 3); };  // query of value v
  // staging: thread (query group, d group) moves 4 queries x 4 d of Q^ (op 0) and dO (op 1, with
  // its low terms when split); with d = 128 every thread takes both operands, with d = 64 half each
  constexpr int NT = 2 * D;
  constexpr int NOP = NT == 256 ? 2 : 1;
  uint2_t fx[NOP][4], fxl[SPL ? 4 : 1];
  float fl = 0.0f, fd = 0.0f;
  // rows go through buffer resources of the step's query head: rows past Sq
  // read as zero with no branch (the host keeps Sq * d * 2 below 2^31)
  const uint32_t head_bytes = (uint32_t)(A.Sq * D * 2);
  auto fetch = [&](int step) {
    const int64_t bh = b * A.H + hk * A.G + step / nqb;
    const int q0 = (int)(qstart + (int64_t)(step % nqb) * QB);
    const rsrc_t rq = make_rsrc(A.q + bh * A.Sq * D, head_bytes);
    const rsrc_t rdo = make_rsrc(A.doh + bh * A.Sq * D, head_bytes);
#pragma unroll
    for (int o = 0; o < NOP; ++o) {
      const int op = NOP == 2 ? o : (int)(threadIdx.x / NT);
      const int t = (int)(threadIdx.x % NT);
      const int qg = t % 8, dg = t / 8;
      const rsrc_t src = op == 0 ? rq : rdo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t off = (uint32_t)((((int64_t)q0 + 4 * qg + i) * D + 4 * dg) * 2);
        fx[o][i] = buf_load8(src, off);
        if (SPL && op == 1) fxl[SPL ? i : 0] = buf_load8(make_rsrc(A.dol + bh * A.Sq * D, head_bytes), off);
      }
    }
    if (threadIdx.x < QB) {
      const int64_t qq = q0 + threadIdx.x;
      const bool ok = qq < A.Sq;
      fl = ok ? A.lse[bh * A.Sq + qq] * 1.4426950408889634f : 0.0f;
      fd = ok && !DV ? A.D[bh * A.Sq + qq] : 0.0f;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int o = 0; o < NOP; ++o) {
      const int op = NOP == 2 ? o : (int)(threadIdx.x / NT);
      const int t = (int)(threadIdx.x % NT);
      const int qg = t % 8, dg = t / 8;
      // [query][d] image: Q^ always, dO for dK; [d][query] image: dO for dV, Q^ for dK
      uint16_t* ra = op == 0 ? Qa : (DV ? nullptr : Oa);
      uint16_t* rb = (op == 1) == DV ? Xb : nullptr;
      if (ra) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<uint2_t*>(ra + (4 * qg + i) * RA + 4 * dg) = fx[o][i];
          if (!DV && SPL && op == 1) *reinterpret_cast<uint2_t*>(Oal + (4 * qg + i) * RA + 4 * dg) = fxl[SPL ? i : 0];
        }
      }
      if (rb) {
        uint2_t tr[4];
        transpose4x4_16(fx[o], tr);
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<uint2_t*>(rb + (4 * dg + j) * RB + 4 * qg) = tr[j];
        if (DV && SPL && op == 1) {
          uint2_t trl[4];
          transpose4x4_16(*reinterpret_cast<const uint2_t(*)[4]>(fxl), trl);
#pragma unroll
          for (int j = 0; j < 4; ++j) *reinterpret_cast<uint2_t*>(Xbl + (4 * dg + j) * RB + 4 * qg) = trl[j];
        }
      }
    }
    if (threadIdx.x < QB) {
      lse_s[threadIdx.x] = fl;
      D_s[threadIdx.x] = fd;
    }
  };
  if (nsteps > 0) fetch(0);
  for (int step = 0; step < nsteps; ++step) {
    const int64_t q0 = qstart + (int64_t)(step % nqb) * QB;
    __syncthreads();  // the previous step's LDS reads are done
    stage();
    if (step + 1 < nsteps) fetch(step + 1);  // in flight during this step's products
    __syncthreads();
    if constexpr (DV) {
      // S^T = K^ Q^T: lane (query r32 of the step, h) holds keys 16h + v of the wave
      float16_t sacc = float16_t{0};
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        sacc = mfma_bf16(kf[s], *reinterpret_cast<const uint4_t*>(Qa + r32 * RA + 16 * s + 8 * hi), sacc);
      const int64_t qq = q0 + r32;
      const int64_t kb = key0 + 32 * wave + 16 * hi;  // this lane's first key
      float x[16];
      const int64_t wkey1 = key0 + 32 * wave + 31;  // the wave's last key
      const bool full = wkey1 < A.Sk && q0 + QB <= A.Sq && (!A.causal || wkey1 <= q0);
      if (full) {
#pragma unroll
        for (int v = 0; v < 16; ++v) x[v] = sacc[v] * A.c;
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const bool vis = kb + v < A.Sk && qq < A.Sq && (!A.causal || kb + v <= qq);
          x[v] = vis ? sacc[v] * A.c : -__builtin_inff();
        }
      }
      // the lane's 16 keys are one level-2 block of its query: block maximum
      // in registers, tile maximum over kv_tile keys through LDS
      const float bm = max16v(x);
      tmx[2 * wave + hi][r32] = bm;
      __syncthreads();
      const int e0 = A.kv_tile == 128 ? 0 : 2 * (wave & 2);
      const int ne = A.kv_tile == 128 ? 8 : 4;
      float tmi = tmx[e0][r32];
      for (int e = 1; e < ne; ++e) tmi = __builtin_fmaxf(tmi, tmx[e0 + e][r32]);
      const bool live = bm != -__builtin_inff();  // a block with no visible key gets scale 0
      const float emax = live ? __builtin_amdgcn_exp2f(bm - tmi) : 0.0f;
      const uint32_t byte = f32_to_e4m3(A.single ? div6_rn(emax) : emax * 448.0f);
      const float2_t fs = ptab[byte];
      const float sh = live ? tmi : 0.0f;
      const float f0 = live ? fs[0] : 0.0f;  // (an empty block: 2^-inf times 0)
      // s2 times the tile weight, rounded once before the product with the code value
      const float s2w =
          live ? fs[1] * (__builtin_amdgcn_exp2f(tmi - lse_s[r32]) * (A.single ? 1.0f : 1.0f / 2688.0f)) : 0.0f;
      float w16[16];
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float t0 = __builtin_amdgcn_exp2f(x[v] - sh) * f0;
        const float t1 = __builtin_amdgcn_exp2f(x[v + 1] - sh) * f0;
        const float2_t cv = cvt_pk_f32_fp4<0>(cvt_pk_fp4<0>(0u, t0, t1));
        w16[v] = cv[0] * s2w;  // (s2 times the weight is rounded once, then the product)
        w16[v + 1] = cv[1] * s2w;
      }
      // hi = the top 16 bits, lo = the rest rounded to bf16 (as pack8), written
      // as [query][key] and read back as the A operand of dV += P^T X: lane
      // (key r32, h) takes queries 16 ks + 8 h .. +8
      uint16_t* ph = pth + (wave * QB + r32) * RPT + 16 * hi;
      uint16_t* pl = ptl + (wave * QB + r32) * RPT + 16 * hi;
#pragma unroll
      for (int hv = 0; hv < 2; ++hv) {
        uint4_t wh, wl;
        pack8<true>(w16 + 8 * hv, wh, wl);
        *reinterpret_cast<uint4_t*>(ph + 8 * hv) = wh;
        *reinterpret_cast<uint4_t*>(pl + 8 * hv) = wl;
      }
      // the wave reads what its own lanes wrote (LDS operations of a wave stay in order)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint16_t* rh = pth + (wave * QB + 16 * ks + 8 * hi) * RPT + r32;
        const uint16_t* rl = ptl + (wave * QB + 16 * ks + 8 * hi) * RPT + r32;
        uint4_t wa, wl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wa[j] = (uint32_t)rh[(2 * j) * RPT] | ((uint32_t)rh[(2 * j + 1) * RPT] << 16);
          wl[j] = (uint32_t)rl[(2 * j) * RPT] | ((uint32_t)rl[(2 * j + 1) * RPT] << 16);
        }
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const int row = (32 * t + r32) * RB + 16 * ks + 8 * hi;
          const uint4_t xb = *reinterpret_cast<const uint4_t*>(Xb + row);
          acc[t] = mfma_bf16(wa, xb, acc[t]);
          acc[t] = mfma_bf16(wl, xb, acc[t]);
          if (SPL) acc[t] = mfma_bf16(wa, *reinterpret_cast<const uint4_t*>(Xbl + row), acc[t]);
        }
      }
    } else {
      // S = Q^ K^T and dP = dO V^T: lane holds key r32 of the wave and the 16 queries qof(v)
      float16_t sacc = float16_t{0}, dp = float16_t{0};
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        sacc = mfma_bf16(*reinterpret_cast<const uint4_t*>(Qa + qr * RA + 16 * s + 8 * hi), kf[s], sacc);
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        dp = mfma_bf16(*reinterpret_cast<const uint4_t*>(Oa + qr * RA + 16 * s + 8 * hi), vf[DV ? 0 : s], dp);
        if (SPL) dp = mfma_bf16(*reinterpret_cast<const uint4_t*>(Oal + qr * RA + 16 * s + 8 * hi), vf[DV ? 0 : s], dp);
      }
      float x[16];
      // every (key, query) pair of the wave's step visible: no mask (the common case)
      const int64_t wkey1 = key0 + 32 * wave + 31;  // the wave's last key
      const bool full = wkey1 < A.Sk && q0 + QB <= A.Sq && (!A.causal || wkey1 <= q0);
      if (full) {
#pragma unroll
        for (int v = 0; v < 16; ++v) x[v] = sacc[v] * A.c;
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t qq = q0 + qof(v);
          const bool vis = kok && qq < A.Sq && (!A.causal || key <= qq);
          x[v] = vis ? sacc[v] * A.c : -__builtin_inff();
        }
      }
      float w16[16];  // dS of this lane's key and queries
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qb = 8 * hi + 16 * h;
        const float4_t la = *reinterpret_cast<const float4_t*>(&lse_s[qb]);
        const float4_t lc = *reinterpret_cast<const float4_t*>(&lse_s[qb + 4]);
        const float4_t da = *reinterpret_cast<const float4_t*>(&D_s[qb]);
        const float4_t dc = *reinterpret_cast<const float4_t*>(&D_s[qb + 4]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          w16[8 * h + j] = A.alpha * __builtin_amdgcn_exp2f(x[8 * h + j] - la[j]) * (dp[8 * h + j] - da[j]);
          w16[8 * h + 4 + j] = A.alpha * __builtin_amdgcn_exp2f(x[8 * h + 4 + j] - lc[j]) * (dp[8 * h + 4 + j] - dc[j]);
        }
      }
      // acc += dS^T Q^: A = this lane's values (k-step ks: values 8 ks .. 8 ks + 7), B = the
      // [d][query] image of Q^
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4_t wa, wl;
        pack8<true>(w16 + 8 * ks, wa, wl);
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const int row = (32 * t + r32) * RB + 16 * ks + 8 * hi;
          const uint4_t xb = *reinterpret_cast<const uint4_t*>(Xb + row);
          acc[t] = mfma_bf16(wa, xb, acc[t]);
          acc[t] = mfma_bf16(wl, xb, acc[t]);
        }
      }
    }
  }
  // lane holds column d = 32 t + r32, rows (keys) 8 (v/4) + 4 h + v%4 of the wave's 32
  float* out = DV ? A.dv : A.dk;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t kk = key0 + 32 * wave + 8 * (v / 4) + 4 * hi + (v % 4);
      if (kk < A.Sk) out[(bhk * A.Sk + kk) * D + 32 * t + r32] = acc[t][v];
    }
}

// ---- dQ without materialized scores -----------------------------------------
//
// One workgroup per 128 query rows (4 waves x 32), looping over key tiles (32
// keys at d = 128, 64 at d = 64), each fetched into registers while the tile
// before it computes.  Per 32-key subtile the wave recomputes S^T = K^ Q^T
// and dP^T = V^ dO^T with K^ and V^ rows fed in the krow2 order, so that
// lane (query, h) holds keys 8h..8h+7 and 16+8h..16+8h+7 -- the k order of
// the B operand of dQ^T += K^T dS^T -- forms dS = s P (dP - D) with
// P = 2^(x - lse2) (dQ needs no P^), and accumulates dQ^T with K^T staged
// transposed in LDS.

struct QArgs {
  const uint16_t *q, *k, *v, *doh, *dol;
  const float *D, *lse;
  float* dq;
  int64_t H, G, Sq, Sk;
  int causal, nqt;
  float c, alpha;
};

template <int D, bool SPLIT_DO>
__global__ void __launch_bounds__(256, 2) bwd_q_kernel(QArgs A) {
  constexpr int KT = 4096 / D;  // keys per tile: one 4 x 4 block of K and of V per thread
  constexpr int RA = D + 8;    // [key][d] rows, bf16
  constexpr int RT = KT + 8;   // [d][key] rows, bf16
  __shared__ uint16_t Ka[KT * RA], Va[KT * RA], Kt[D * RT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hi = lane >> 5, r32 = lane & 31;
  const int64_t BH = gridDim.x / A.nqt;
  const int64_t gi = blockIdx.x;
  const int64_t bh = gi % BH, qrank = gi / BH;  // heads interleaved, the heaviest causal rows first
  const int qt = (int)(A.causal ? A.nqt - 1 - qrank : qrank);
  const int64_t b = bh / A.H, h = bh - b * A.H;
  const int64_t bhk = b * (A.H / A.G) + h / A.G;
  const int64_t q = (int64_t)qt * kGT + 32 * wave + r32;
  const bool qok = q < A.Sq;
  const int64_t qidx = bh * A.Sq + (qok ? q : 0);
  uint4_t qf[D / 16], df[D / 16], dl[SPLIT_DO ? D / 16 : 1];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = fragb(A.q + qidx * D + 16 * s + 8 * hi, qok);
    df[s] = fragb(A.doh + qidx * D + 16 * s + 8 * hi, qok);
    if (SPLIT_DO) dl[SPLIT_DO ? s : 0] = fragb(A.dol + qidx * D + 16 * s + 8 * hi, qok);
  }
  const float lse2 = qok ? A.lse[qidx] * 1.4426950408889634f : 0.0f;
  const float Dq = qok ? A.D[qidx] : 0.0f;
  float16_t acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc[t] = float16_t{0};
  const int64_t qend = ((int64_t)qt + 1) * kGT;
  const int64_t kend = A.causal && qend < A.Sk ? qend : A.Sk;
  const int ntile = (int)((kend + KT - 1) / KT);
  const uint16_t* kb = A.k + bhk * A.Sk * D;
  const uint16_t* vb = A.v + bhk * A.Sk * D;
  const int kr = krow2(r32);
  // K^ and V^ rows of a tile, fetched into registers one tile ahead (thread
  // (key group, d group) moves 4 keys x 4 d of each) and staged as [key][d]
  // images and a [d][key] image of K^
  constexpr int NU = KT * D / 16 / 256;
  uint2_t xk[NU][4], xv[NU][4];
  // rows through buffer resources of the kv head: keys past Sk read as zero
  // with no branch (the host keeps Sk * d * 2 below 2^31)
  const rsrc_t rk = make_rsrc(kb, (uint32_t)(A.Sk * D * 2)), rv = make_rsrc(vb, (uint32_t)(A.Sk * D * 2));
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int id = (int)threadIdx.x + 256 * u;
      const int kg = id % (KT / 4), dg = id / (KT / 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t off = (uint32_t)(((k0 + 4 * kg + i) * D + 4 * dg) * 2);
        xk[u][i] = buf_load8(rk, off);
        xv[u][i] = buf_load8(rv, off);
      }
    }
  };
  if (ntile > 0) fetch(0);
  for (int tile = 0; tile < ntile; ++tile) {
    const int64_t key0 = (int64_t)tile * KT;
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int id = (int)threadIdx.x + 256 * u;
      const int kg = id % (KT / 4), dg = id / (KT / 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint2_t*>(Ka + (4 * kg + i) * RA + 4 * dg) = xk[u][i];
        *reinterpret_cast<uint2_t*>(Va + (4 * kg + i) * RA + 4 * dg) = xv[u][i];
      }
      uint2_t tr[4];
      transpose4x4_16(xk[u], tr);
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<uint2_t*>(Kt + (4 * dg + j) * RT + 4 * kg) = tr[j];
    }
    if (tile + 1 < ntile) fetch(key0 + KT);  // in flight during this tile's products
    __syncthreads();
#pragma unroll
    for (int g = 0; g < KT / 32; ++g) {
      float16_t s = float16_t{0}, dp = float16_t{0};
      const uint16_t* ka = Ka + (32 * g + kr) * RA + 8 * hi;
      const uint16_t* va = Va + (32 * g + kr) * RA + 8 * hi;
#pragma unroll
      for (int k = 0; k < D / 16; ++k) s = mfma_bf16(*reinterpret_cast<const uint4_t*>(ka + 16 * k), qf[k], s);
#pragma unroll
      for (int k = 0; k < D / 16; ++k) {
        const uint4_t a = *reinterpret_cast<const uint4_t*>(va + 16 * k);
        dp = mfma_bf16(a, df[k], dp);
        if (SPLIT_DO) dp = mfma_bf16(a, dl[k], dp);
      }
      float ds[16];
      // every (key, query) pair of the wave's subtile visible: no mask (the common case; with
      // the split dO the second copy of the loop would not fit the registers)
      const int64_t skey1 = key0 + 32 * g + 31, wq0 = q - r32;
      if (!SPLIT_DO && wq0 + 32 <= A.Sq && skey1 < A.Sk && (!A.causal || skey1 <= wq0)) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          ds[v] = A.alpha * __builtin_amdgcn_exp2f(s[v] * A.c - lse2) * (dp[v] - Dq);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t key = key0 + 32 * g + (v & 7) + 8 * hi + 16 * (v >> 3);
          const bool vis = qok && key < A.Sk && (!A.causal || key <= q);
          const float x = vis ? s[v] * A.c : -__builtin_inff();
          ds[v] = A.alpha * __builtin_amdgcn_exp2f(x - lse2) * (dp[v] - Dq);  // P masked: 0
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4_t da, dlo;
        pack8<true>(ds + 8 * ks, da, dlo);
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const uint4_t a = *reinterpret_cast<const uint4_t*>(Kt + (32 * t + r32) * RT + 32 * g + 16 * ks + 8 * hi);
          acc[t] = mfma_bf16(a, da, acc[t]);
          acc[t] = mfma_bf16(a, dlo, acc[t]);
        }
      }
    }
  }
  // dQ^T: lane column = this query, rows d = 32 t + 8 (v/4) + 4 h + v%4
  if (qok) {
    float* dst = A.dq + (bh * A.Sq + q) * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4_t*>(dst + 32 * t + 8 * j + 4 * hi) =
            float4_t{acc[t][4 * j], acc[t][4 * j + 1], acc[t][4 * j + 2], acc[t][4 * j + 3]};
  }
}

}  // namespace fp4dev

using namespace fp4dev;

size_t fp4i_attn_bwd_workspace(const AttnBwdLaunch& L) {
  auto a = [](size_t n) { return (n + 255) & ~(size_t)255; };
  const size_t nq = (size_t)(L.B * L.H * L.Sq), nk = (size_t)(L.B * L.Hkv * L.Sk);
  // bf16 Q^, K^, V^; the two bf16 terms of an fp16 dO; D
  return a(nq * L.d * 2) * 3 + a(nk * L.d * 2) * 2 + a(nq * 4);
}

hipError_t fp4i_launch_attn_bwd(const AttnBwdLaunch& L, hipStream_t st) {
  auto a = [](size_t n) { return (n + 255) & ~(size_t)255; };
  const int64_t B = L.B, H = L.H, Hkv = L.Hkv, Sq = L.Sq, Sk = L.Sk, d = L.d, G = H / Hkv;
  const size_t nq = (size_t)(B * H * Sq), nk = (size_t)(B * Hkv * Sk);
  const bool fp16_do = L.dtype == 1;  // dO in fp16 is not a bf16 number: split it
  char* w = (char*)L.ws;
  uint16_t* qh = (uint16_t*)w; w += a(nq * d * 2);
  uint16_t* doh = (uint16_t*)w; w += a(nq * d * 2);
  uint16_t* dol = (uint16_t*)w; w += a(nq * d * 2);
  uint16_t* kh = (uint16_t*)w; w += a(nk * d * 2);
  uint16_t* vh = (uint16_t*)w; w += a(nk * d * 2);
  float* Dv = (float*)w;
  auto blocks = [](int64_t n) { return dim3((unsigned)((n + 255) / 256)); };
  // operands
  hipLaunchKernelGGL(dequant_rows_kernel, blocks((int64_t)nq * d / 8), dim3(256), 0, st, L.qc, L.qs, (int64_t)nq,
                     (int)d, qh);
  hipLaunchKernelGGL(dequant_rows_kernel, blocks((int64_t)nk * d / 8), dim3(256), 0, st, L.kc, L.ks, (int64_t)nk,
                     (int)d, kh);
  hipLaunchKernelGGL(dequant_cols_kernel, blocks((int64_t)nk / 2 * d), dim3(256), 0, st, L.vc, L.vs, (int64_t)nk,
                     (int)d, vh);
  const uint16_t* dO_hi = (const uint16_t*)L.dout;  // a bf16 dO is used as it is
  const uint16_t* dO_lo = nullptr;
  if (fp16_do) {
    hipLaunchKernelGGL(split_f16_kernel, blocks((int64_t)nq * d), dim3(256), 0, st, (const half_t*)L.dout,
                       (int64_t)nq * d, doh, dol);
    dO_hi = doh;
    dO_lo = dol;
  }
  const dim3 rd((unsigned)((nq + 15) / 16));
  if (fp16_do) {
    const half_t* dO = (const half_t*)L.dout;
    if (L.hp_dtype == 2) hipLaunchKernelGGL((row_dot_kernel<half_t, float>), rd, dim3(256), 0, st, dO, (const float*)L.out_hp, (int64_t)nq, (int)d, Dv);
    else if (L.hp_dtype == 1) hipLaunchKernelGGL((row_dot_kernel<half_t, half_t>), rd, dim3(256), 0, st, dO, (const half_t*)L.out_hp, (int64_t)nq, (int)d, Dv);
    else hipLaunchKernelGGL((row_dot_kernel<half_t, uint16_t>), rd, dim3(256), 0, st, dO, (const uint16_t*)L.out_hp, (int64_t)nq, (int)d, Dv);
  } else {
    const uint16_t* dO = (const uint16_t*)L.dout;
    if (L.hp_dtype == 2) hipLaunchKernelGGL((row_dot_kernel<uint16_t, float>), rd, dim3(256), 0, st, dO, (const float*)L.out_hp, (int64_t)nq, (int)d, Dv);
    else if (L.hp_dtype == 1) hipLaunchKernelGGL((row_dot_kernel<uint16_t, half_t>), rd, dim3(256), 0, st, dO, (const half_t*)L.out_hp, (int64_t)nq, (int)d, Dv);
    else hipLaunchKernelGGL((row_dot_kernel<uint16_t, uint16_t>), rd, dim3(256), 0, st, dO, (const uint16_t*)L.out_hp, (int64_t)nq, (int)d, Dv);
  }
  const float alpha = L.c * 0.69314718055994531f;  // s = c ln 2
  // dQ per 128 query rows
  QArgs qa;
  qa.q = qh; qa.k = kh; qa.v = vh; qa.doh = dO_hi; qa.dol = dO_lo; qa.D = Dv; qa.lse = L.lse;
  qa.dq = L.dq;
  qa.H = H; qa.G = G; qa.Sq = Sq; qa.Sk = Sk;
  qa.causal = L.causal;
  qa.nqt = (int)((Sq + kGT - 1) / kGT);
  qa.c = L.c;
  qa.alpha = alpha;
  const dim3 qgrid((unsigned)(B * H * qa.nqt));
  if (d == 128) {
    if (fp16_do) hipLaunchKernelGGL((bwd_q_kernel<128, true>), qgrid, dim3(256), 0, st, qa);
    else hipLaunchKernelGGL((bwd_q_kernel<128, false>), qgrid, dim3(256), 0, st, qa);
  } else {
    if (fp16_do) hipLaunchKernelGGL((bwd_q_kernel<64, true>), qgrid, dim3(256), 0, st, qa);
    else hipLaunchKernelGGL((bwd_q_kernel<64, false>), qgrid, dim3(256), 0, st, qa);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dK and dV per key tile, over the G query heads of each kv head
  KvArgs ka;
  ka.q = qh; ka.k = kh; ka.v = vh; ka.doh = dO_hi; ka.dol = dO_lo; ka.D = Dv; ka.lse = L.lse;
  ka.dk = L.dk; ka.dv = L.dv;
  ka.H = H; ka.G = G; ka.Sq = Sq; ka.Sk = Sk;
  ka.kv_tile = L.kv_tile; ka.causal = L.causal; ka.single = L.single;
  ka.nkt = (int)((Sk + kGT - 1) / kGT);
  ka.c = L.c;
  ka.alpha = alpha;
  const dim3 kgrid((unsigned)(B * Hkv * ka.nkt));
  if (d == 128) {
    if (fp16_do) {
      hipLaunchKernelGGL((bwd_kv_kernel<128, true, 0>), kgrid, dim3(256), 0, st, ka);
      hipLaunchKernelGGL((bwd_kv_kernel<128, true, 1>), kgrid, dim3(256), 0, st, ka);
    } else {
      hipLaunchKernelGGL((bwd_kv_kernel<128, false, 0>), kgrid, dim3(256), 0, st, ka);
      hipLaunchKernelGGL((bwd_kv_kernel<128, false, 1>), kgrid, dim3(256), 0, st, ka);
    }
  } else {
    if (fp16_do) {
      hipLaunchKernelGGL((bwd_kv_kernel<64, true, 0>), kgrid, dim3(256), 0, st, ka);
      hipLaunchKernelGGL((bwd_kv_kernel<64, true, 1>), kgrid, dim3(256), 0, st, ka);
    } else {
      hipLaunchKernelGGL((bwd_kv_kernel<64, false, 0>), kgrid, dim3(256), 0, st, ka);
      hipLaunchKernelGGL((bwd_kv_kernel<64, false, 1>), kgrid, dim3(256), 0, st, ka);
    }
  }
  return hipGetLastError();
}

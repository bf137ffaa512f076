// attn_fwd.hip -- fused FP4 attention forward for gfx950 (CDNA4).
//
// What it computes (ScaleSearch page, Metodologia / ScaleSearchAttention:
// QK^T and PV on NVFP4 operands with FP32 accumulation; ThriftAttention page,
// Metodologia / 2: FP4 path with two-level quantization of P for most block
// pairs, FP16 path for the selected ones, both merged by an online softmax):
//   for every query row i and key tile T (kv_tile keys):
//     x = fl32(S * c), tm = max over visible keys, e = 2^(x - tm)
//     FP4 tile:  16-key blocks of e get s2 = E4M3(amax(e) * 448), codes
//                RNE_E2M1(e * fl32(2688/s2)), P^ = code * s2; the tile adds
//                (P^ V^) / 2688 with weight 2^(tm - m)
//     FP16 tile: adds fp16(e) fp16(V) (scores from fp16 q and k)
//     l sums the unquantized e; out = O / l.
//   Single-level P (Attn-QAT page, Metodologia / B, option): the FP4 tile's
//   blocks take s2 = E4M3(amax(e) / 6) and codes RNE_E2M1(e / s2) directly,
//   and the tile adds P^ V^ (no row level).
//
// MI355X mapping.  gfx950's block-scaled FP4 MFMA takes power-of-two scales
// per 32 elements, while NVFP4 scales are E4M3 per 16, so the operands are
// dequantized exactly to fp16 (code * scale has at most 6 significant bits)
// and run on v_mfma_f32_32x32x16_f16.  One workgroup = 4 waves = 128 query
// rows of one (batch, head); a wave owns 32 rows.  Per key tile:
//   - all 256 lanes dequantize the tile's K and V codes into LDS (K as
//     [key][d], V transposed as [d][key]); the next tile's codes are fetched
//     into registers while the current tile computes;
//   - each wave computes S^T = K Q^T (32 keys x 32 queries per MFMA tile).  K
//     rows are fed in a permuted order so that every lane ends up holding one
//     query row's 16 consecutive keys: the level-2 P scale is a lane-local
//     reduction, only the tile row maximum crosses to lane ^ 32;
//   - P stays in registers and is the B operand of O^T += V^T P^T; V's LDS
//     layout uses the matching key order, so P needs no shuffle.
// The FP4 tiles run first, the FP16 tiles after (their fp16 Q fragment is
// loaded only when a selected pair exists), as the ThriftAttention page does
// to limit register pressure.  A wave raises its issue priority while it runs
// an MFMA loop, so that on a SIMD shared by two workgroups the MFMA stream
// of one wave keeps going while the other wave's softmax fills the VALU.
#include "device_common.h"
#include "fp4_internal.h"

namespace fp4dev {

// Natural logarithm in double precision for compile-time tables: x = 2^k y
// with y in [1, 2), ln y = 2 atanh((y - 1) / (y + 1)) by its power series
// (|z| <= 1/3, so 40 terms are far past double precision).
constexpr double ct_ln(double x) {
  int k = 0;
  while (x >= 2.0) { x /= 2.0; ++k; }
  while (x < 1.0) { x *= 2.0; --k; }
  const double z = (x - 1.0) / (x + 1.0), z2 = z * z;
  double term = z, sum = 0.0;
  for (int n = 0; n < 40; ++n) {
    sum += term / (2 * n + 1);
    term *= z2;
  }
  return 2.0 * sum + k * 0.69314718055994530942;
}

// Level-2 P scale data for every E4M3 scale byte s2 (compile-time):
//   lg  = log2(2688 / s2), so the level-2 quantization input e * 2688 / s2 is
//         formed as 2^(x - tm + lg) in one exponential;
//   inv = s2 / 2688, which turns a block's sum of those inputs back into the
//         sum of its unquantized e for the softmax denominator;
//   s   = s2 itself.
// Byte 0 (a block whose largest e is below half the smallest E4M3 step) has
// s2 = 0: lg = 0 and inv = 1, so its inputs are the plain e (all of which
// quantize to code 0) and its denominator sum is still the sum of e.
struct PScaleTable {
  float4_t v[128];  // {lg, inv, s, 0}
  constexpr PScaleTable() : v() {
    for (int b = 0; b < 128; ++b) {
      double s2 = 0.0;
      if (b < 8) s2 = (double)b / 512.0;
      else {
        int e = (b >> 3) - 7, mm = b & 7;
        s2 = 1.0 + (double)mm / 8.0;
        for (int i = 0; i < e; ++i) s2 *= 2.0;
        for (int i = 0; i > e; --i) s2 /= 2.0;
      }
      if (b == 0 || b == 127) v[b] = float4_t{0.0f, 1.0f, 0.0f, 0.0f};
      else v[b] = float4_t{(float)(ct_ln(2688.0 / s2) / 0.69314718055994530942), (float)(s2 / 2688.0), (float)s2, 0.0f};
    }
  }
};
__constant__ PScaleTable kPScale = PScaleTable();

// Single-level P (Attn-QAT page, Metodologia / B: no two-level step): the
// block scale is s2 = E4M3(max e / 6) itself, so lg = log2(1 / s2), inv = s2
// and s = s2; the tile adds P^ V^ with P^ in units of e.
struct PScaleTable1 {
  float4_t v[128];  // {lg, inv, s, 0}
  constexpr PScaleTable1() : v() {
    for (int b = 0; b < 128; ++b) {
      double s2 = 0.0;
      if (b < 8) s2 = (double)b / 512.0;
      else {
        int e = (b >> 3) - 7, mm = b & 7;
        s2 = 1.0 + (double)mm / 8.0;
        for (int i = 0; i < e; ++i) s2 *= 2.0;
        for (int i = 0; i > e; --i) s2 /= 2.0;
      }
      if (b == 0 || b == 127) v[b] = float4_t{0.0f, 1.0f, 0.0f, 0.0f};
      else v[b] = float4_t{(float)(ct_ln(1.0 / s2) / 0.69314718055994530942), (float)s2, (float)s2, 0.0f};
    }
  }
};
__constant__ PScaleTable1 kPScale1 = PScaleTable1();

constexpr int kWaves = 4;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup

// Value of lane ^ 32, with v_permlane32_swap (a VALU op: no LDS round trip).
// Called with the same register as both operands, the swap returns the
// lower half's values in the upper lanes of the first result and the upper
// half's values in the lower lanes of the second.
__device__ __forceinline__ float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Position of key k (within a 32-key group) in the V^T LDS row: the 8-key
// groups 1 and 2 trade places, matching the keys each lane holds in S^T.
__device__ __forceinline__ int vpos(int k) { return (k & ~31) | ((k & 8) << 1) | ((k & 16) >> 1) | (k & 7); }

// A-operand row of S^T for key k inside a 32-key subtile, inverse of the
// MFMA output row -> key map key(row) = (row%4) + 4*(row/8) + 16*((row/4)%2).
__device__ __forceinline__ int krow_of_lane(int r) { return (r & 3) | ((r >> 3) << 2) | (((r >> 2) & 1) << 4); }

template <typename OT>
__device__ __forceinline__ void store4(OT* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4_t*>(p) = float4_t{a, b, c, d};
}
template <>
__device__ __forceinline__ void store4<half_t>(half_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<half4_t*>(p) = half4_t{(half_t)a, (half_t)b, (half_t)c, (half_t)d};
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  uint2_t w;
  w[0] = (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
  w[1] = (uint32_t)f32_to_bf16_rne(c) | ((uint32_t)f32_to_bf16_rne(d) << 16);
  *reinterpret_cast<uint2_t*>(p) = w;
}

// fp16 (RNE) of a bf16 or fp16 input element pair packed in a dword.
template <typename IT>
__device__ __forceinline__ half2_t to_half2(uint32_t w);
template <>
__device__ __forceinline__ half2_t to_half2<uint16_t>(uint32_t w) {
  return half2_t{(half_t)__uint_as_float(w << 16), (half_t)__uint_as_float(w & 0xFFFF0000u)};
}
template <>
__device__ __forceinline__ half2_t to_half2<half_t>(uint32_t w) {
  return __builtin_bit_cast(half2_t, w);
}

// LDS tiles are declared in 16-byte units so that every fragment read is a
// single ds_read_b128 with an immediate offset.  Bank rules of the gfx950 LDS
// (measured with the bank-conflict counter): a 16-byte read is conflict-free
// when each half-wave's distinct 16-byte units differ mod 32; a 4-byte write
// when each half-wave's dwords differ mod 32; a 16-byte write when each group
// of 8 lanes' units differ mod 8.  Rows carry one unit of padding (K and V^T
// fragment reads), and V^T rows of d-group c = d / 16 shift by vpad(c) units
// so that the staging writes, whose half-waves cover d-groups 32 rows apart,
// spread over all banks.  vpad is equal within each 32-row block (reads keep
// a lane-independent offset) and never decreases (rows never overlap).
template <int D, int BC>
struct Smem {
  static constexpr int KS8 = D / 8 + 1;   // 16-byte units per K row (one unit of pad)
  static constexpr int VS8 = BC / 8 + 1;  // 16-byte units per V^T row
  static __device__ __forceinline__ constexpr int vpad(int grp) {
    return D == 128 ? 4 * (grp >> 2) + ((grp >> 1) & 1) : 4 * (grp >> 1);
  }
  // V^T row of d = r + 32 t (r < 32): r * VS8 + vrow_t(t)
  static __device__ __forceinline__ constexpr int vrow_t(int t) { return 32 * t * VS8 + vpad(2 * t); }
  half8_t k[BC * KS8];
  half8_t v[D * VS8 + 16];
  float4_t pt[128];  // level-2 P scale data, indexed by the E4M3 byte
};

// Which 16-byte chunk of the tile's codes each thread fetches and stages.
// K chunk: key row kr, 32-column block dc; a group of 8 lanes takes 8 rows of
// one block (16-byte LDS writes).  V chunk: token pair pr, 16-column block cc;
// a half-wave takes 64/(D/16) pairs of every other block, so its d rows are
// 32 apart (4-byte LDS writes).  Either way a wave reads whole rows of codes.
template <int D>
struct StageMap {
  static constexpr int NDC = D / 32, NCC = D / 16, PPW = 64 / NCC;
  static __device__ __forceinline__ int k_row(int wv, int l, int u) {
    return (l & 7) + 8 * ((l >> 3) / NDC) + (64 / NDC) * (wv + 4 * u);
  }
  static __device__ __forceinline__ int k_dc(int l) { return (l >> 3) % NDC; }
  static __device__ __forceinline__ int v_pair(int wv, int l, int u) { return PPW * (wv + 4 * u) + (l & 31) % PPW; }
  static __device__ __forceinline__ int v_cc(int l) { return (l >> 5) + 2 * ((l & 31) / PPW); }
};

// One tile's worth of quantized K/V held in registers between fetch and stage.
template <int D, int BC>
struct Fetch {
  static constexpr int NCH = BC * D / 32;               // 16-byte chunks per operand
  static constexpr int PER = (NCH + 255) / 256;          // chunks per thread
  uint4_t kc[PER];
  uint32_t ks[PER];  // two scale bytes (d blocks 2j, 2j+1)
  uint4_t vc[PER];
  uint4_t vs[PER];
};

// Buffer resources of one (batch, kv head): quantized K and V.
struct HeadBufs {
  rsrc_t kc, ks, vc, vs;
};

struct Problem {
  int64_t H, Hkv, Sq, Sk;
  const uint8_t *qc, *qs, *kc, *ks, *vc, *vs;
  const void *q, *k, *v;
  TokMap qmap, kmap, vmap;  // token rows of q, k, v (the FP16 path)
  const int32_t *idx, *cnt;
  int causal, pct, sel_block, nqb, kmax, nqt;
  int xcd_heads;  // workgroup order: whole heads per XCD (else heads interleaved)
  float c;
  void* out;
  float* lse;
};

// Tile loads go through buffer resources: keys past Sk read as zero codes
// (their scores are masked), and no branch or clamp sits between the loads,
// so the next tile's codes stay in flight while the current tile computes.
template <int D, int BC>
__device__ __forceinline__ void fetch_k(Fetch<D, BC>& F, const HeadBufs& hb, int64_t key0) {
  using M = StageMap<D>;
  const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < Fetch<D, BC>::PER; ++u) {
    const int kr = M::k_row(wv, l, u), dc = M::k_dc(l);
    if (Fetch<D, BC>::NCH % 256 == 0 || kr < BC) {  // every thread has a chunk when NCH is a multiple of 256
      const uint32_t key = (uint32_t)key0 + kr;
      F.kc[u] = buf_load16(hb.kc, key * (D / 2) + dc * 16);
      F.ks[u] = buf_load2(hb.ks, key * (D / 16) + dc * 2);
    }
  }
}

template <int D, int BC>
__device__ __forceinline__ void fetch_v(Fetch<D, BC>& F, const HeadBufs& hb, int64_t key0) {
  using M = StageMap<D>;
  const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < Fetch<D, BC>::PER; ++u) {
    const int pr = M::v_pair(wv, l, u), cc = M::v_cc(l);
    if (Fetch<D, BC>::NCH % 256 == 0 || pr < BC / 2) {
      const uint32_t pair = (uint32_t)(key0 / 2) + pr;
      F.vc[u] = buf_load16(hb.vc, pair * D + cc * 16);
      F.vs[u] = buf_load16(hb.vs, (pair / 8) * D + cc * 16);
    }
  }
}

__device__ __forceinline__ half2_t scale_pair(half2_t v, half_t s) { return v * half2_t{s, s}; }

// Two E4M3 scale bytes (bits 0..15 of w) -> two fp16 values (exact).
__device__ __forceinline__ half2_t e4m3x2_to_half2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}
__device__ __forceinline__ half2_t e4m3x2_hi_to_half2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
}

// 8 E2M1 codes (one dword) times one fp16 scale -> 8 fp16 values.
__device__ __forceinline__ half8_t deq8(uint32_t cw, half_t s) {
  half2_t a = scale_pair(cvt_pk_f16_fp4<0>(cw), s), b = scale_pair(cvt_pk_f16_fp4<1>(cw), s);
  half2_t c = scale_pair(cvt_pk_f16_fp4<2>(cw), s), d = scale_pair(cvt_pk_f16_fp4<3>(cw), s);
  return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int D, int BC>
__device__ __forceinline__ void stage_k(const Fetch<D, BC>& F, Smem<D, BC>& S) {
  using M = StageMap<D>;
  const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < Fetch<D, BC>::PER; ++u) {
    const int kr = M::k_row(wv, l, u), dc = M::k_dc(l);
    if (Fetch<D, BC>::NCH % 256 == 0 || kr < BC) {  // every thread has a chunk when NCH is a multiple of 256
      const half2_t ks2 = e4m3x2_to_half2(F.ks[u]);
      half8_t* dst = S.k + kr * Smem<D, BC>::KS8 + dc * 4;
#pragma unroll
      for (int w = 0; w < 4; ++w) dst[w] = deq8(F.kc[u][w], w < 2 ? ks2[0] : ks2[1]);
    }
  }
}

// Word w of V chunk u (four columns of a token pair): byte j of the code word
// is column 16*cc + 4*w + j, tokens (2*pr, 2*pr+1).
template <int D, int BC>
__device__ __forceinline__ void stage_v_word(const Fetch<D, BC>& F, Smem<D, BC>& S, int u, int w) {
  using M = StageMap<D>;
  const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int pr = M::v_pair(wv, l, u), cc = M::v_cc(l);
  if (Fetch<D, BC>::NCH % 256 == 0 || pr < BC / 2) {
    half2_t* v2 = reinterpret_cast<half2_t*>(S.v);
    const int pos = vpos(2 * pr);
    const uint32_t cw = F.vc[u][w], sw = F.vs[u][w];
    const half2_t sa = e4m3x2_to_half2(sw), sb = e4m3x2_hi_to_half2(sw);
    const int col = 16 * cc + 4 * w;
    constexpr int VS2 = Smem<D, BC>::VS8 * 4;  // half2 units per V^T row
    half2_t* dst = v2 + col * VS2 + 4 * Smem<D, BC>::vpad(cc) + pos / 2;
    dst[0 * VS2] = scale_pair(cvt_pk_f16_fp4<0>(cw), sa[0]);
    dst[1 * VS2] = scale_pair(cvt_pk_f16_fp4<1>(cw), sa[1]);
    dst[2 * VS2] = scale_pair(cvt_pk_f16_fp4<2>(cw), sb[0]);
    dst[3 * VS2] = scale_pair(cvt_pk_f16_fp4<3>(cw), sb[1]);
  }
}

template <int D, int BC>
__device__ __forceinline__ void stage_v(const Fetch<D, BC>& F, Smem<D, BC>& S) {
#pragma unroll
  for (int u = 0; u < Fetch<D, BC>::PER; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) stage_v_word<D, BC>(F, S, u, w);
}

// FP16 path: the original bf16/fp16 K and V of one step of keys (32 at
// d = 128, 64 at d = 64: the most whose registers fit beside the wave's
// state), fetched into registers (buffer loads, so keys past Sk read as zero)
// one step ahead of their use and then converted to fp16 into the first keys
// of the tile layout.  K: rows x D, 16 bytes per load.  V: a chunk is a token
// pair x 8 columns going to V^T; as in the FP4 staging, a half-wave's chunks
// sit in d-groups 32 rows apart (conflict-free writes).
template <int D>
constexpr int kStepKeys = D == 128 ? 32 : 64;

template <int D>
struct Fetch16 {
  static constexpr int NK = kStepKeys<D>;
  static constexpr int NKU = NK * D / 8 / 256;         // K loads per thread
  static constexpr int NVU = (NK / 2) * (D / 8) / 256;  // V chunks per thread (two loads each)
  static_assert(NKU * 256 == NK * D / 8 && NVU * 256 == (NK / 2) * (D / 8) && NVU >= 1, "whole rounds");
  uint4_t k[NKU];
  uint4_t v0[NVU], v1[NVU];
};

template <int D>
struct Stage16Map {
  static constexpr int PPW = 1024 / D;  // token pairs per half-wave row of chunks
  static __device__ __forceinline__ int k_row(int u) { return (threadIdx.x + 256 * u) / (D / 8); }
  static __device__ __forceinline__ int k_dc(int u) { return (threadIdx.x + 256 * u) % (D / 8); }
  static __device__ __forceinline__ int v_pair(int it) {
    const int z = (threadIdx.x >> 6) + 4 * it, lp = threadIdx.x & 31;
    return PPW * (z >> 1) + lp % PPW;
  }
  static __device__ __forceinline__ int v_grp() { return ((threadIdx.x & 63) >> 5) + 2 * ((threadIdx.x & 31) / PPW); }
  static __device__ __forceinline__ int v_c8(int it) { return 2 * v_grp() + ((((threadIdx.x >> 6) + 4 * it)) & 1); }
};

// kts, vts: elements between consecutive tokens of K and V
template <int D>
__device__ __forceinline__ void fetch16(Fetch16<D>& G, rsrc_t kr16, rsrc_t vr16, uint32_t kts, uint32_t vts,
                                        int64_t key0) {
  using M = Stage16Map<D>;
#pragma unroll
  for (int u = 0; u < Fetch16<D>::NKU; ++u) {
    const uint32_t key = (uint32_t)key0 + M::k_row(u);
    G.k[u] = buf_load16(kr16, (key * kts + M::k_dc(u) * 8) * 2);
  }
#pragma unroll
  for (int it = 0; it < Fetch16<D>::NVU; ++it) {
    const uint32_t key = (uint32_t)key0 + 2 * M::v_pair(it);
    const int c8 = M::v_c8(it);
    G.v0[it] = buf_load16(vr16, (key * vts + c8 * 8) * 2);
    G.v1[it] = buf_load16(vr16, ((key + 1) * vts + c8 * 8) * 2);
  }
}

template <int D, int BC, typename IT>
__device__ __forceinline__ void stage16(const Fetch16<D>& G, Smem<D, BC>& S) {
  using M = Stage16Map<D>;
#pragma unroll
  for (int u = 0; u < Fetch16<D>::NKU; ++u) {
    const uint4_t w = G.k[u];
    half2_t a = to_half2<IT>(w[0]), b = to_half2<IT>(w[1]), c = to_half2<IT>(w[2]), d2 = to_half2<IT>(w[3]);
    S.k[M::k_row(u) * Smem<D, BC>::KS8 + M::k_dc(u)] = half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d2[0], d2[1]};
  }
  half2_t* v2 = reinterpret_cast<half2_t*>(S.v);
  constexpr int VS2 = Smem<D, BC>::VS8 * 4;
#pragma unroll
  for (int it = 0; it < Fetch16<D>::NVU; ++it) {
    const int pos = vpos(2 * M::v_pair(it));
    half2_t* dst = v2 + 8 * M::v_c8(it) * VS2 + 4 * Smem<D, BC>::vpad(M::v_grp()) + pos / 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half2_t a = to_half2<IT>(G.v0[it][j]), b = to_half2<IT>(G.v1[it][j]);
      dst[(2 * j) * VS2] = half2_t{a[0], b[0]};
      dst[(2 * j + 1) * VS2] = half2_t{a[1], b[1]};
    }
  }
}

// Per-wave state.  The output accumulator U and the denominator l are kept
// relative to a per-row reference exponent m: the true unnormalized output is
// U * 2^m.  m is a lazily raised running maximum: it moves only when a tile's
// maximum exceeds it by more than kRaise, so a tile's weight r = 2^(tm - m)
// stays <= 2^kRaise.  FP4 tiles fold r into the fp16 block scale of P^
// (P^ r = code * fp16(s2 * r)) and add P^ V^ with P^ in units of e/2688 (of
// e with single-level P); the switch to FP16 tiles rescales U to units of e
// once.  FP16 tiles take
// p = 2^(x - m) = e r directly.  Either way the PV MFMA accumulates straight
// into U.
template <int D>
struct RowState {
  float16_t o[D / 32];  // U^T: d rows (i%4)+8(i/4)+4(lane/32) of each 32-row group, query lane%32
  float m;              // reference exponent (x units), shared by lanes l and l^32
  float l;              // this lane's part of the denominator
};

// The reference is raised when a tile maximum is more than 2^4 above it
// (keeps code * s2 * r <= 2688 * 16 inside fp16); tiles more than 2^64 below
// it weigh less than 2^-64 of the row and are left out.
constexpr float kRaise = 4.0f;
constexpr float kSkipBelow = 64.0f;

__device__ __forceinline__ float max16(const float16_t& a) {
  float m0 = __builtin_fmaxf(__builtin_fmaxf(a[0], a[1]), a[2]);
  float m1 = __builtin_fmaxf(__builtin_fmaxf(a[3], a[4]), a[5]);
  float m2 = __builtin_fmaxf(__builtin_fmaxf(a[6], a[7]), a[8]);
  float m3 = __builtin_fmaxf(__builtin_fmaxf(a[9], a[10]), a[11]);
  float m4 = __builtin_fmaxf(__builtin_fmaxf(a[12], a[13]), a[14]);
  m0 = __builtin_fmaxf(__builtin_fmaxf(m0, m1), m2);
  m3 = __builtin_fmaxf(__builtin_fmaxf(m3, m4), a[15]);
  return __builtin_fmaxf(m0, m3);
}

// One tile for one wave, in two phases.  FP4: two-level P; else fp16(2^(x - m)).
//
// Scores stay raw (S = q.k) until the exponential: with c > 0 the largest
// fl32(S c) is fl32(max(S) c), so the tile maximum is taken on raw scores and
// each exponent is one fused x*c - offset.  Each lane holds 16 consecutive
// keys of one query row per 32-key subtile, i.e. exactly one level-2 block of
// P, so the block scale is lane-local.
//
// NK: keys processed, the first NK of the tile's LDS layout (the FP16 path
// runs steps of 32 or 64 keys).
template <int NG>
struct ScoreTile {
  float16_t acc[NG];  // S^T of the wave's rows, 32 keys per subtile
  float bmax[NG];     // this lane's block maximum (raw scores) per subtile
};

// Scores: S^T = K Q^T, one 32-key subtile at a time; the mask-and-max of the
// previous subtile runs on the VALU while this subtile's MFMAs execute.  VST:
// this thread's share of the tile's V staging (from F) also runs between the
// MFMAs, in issue slots the scores leave free (the caller orders it before
// the P V phase with a barrier).
template <int D, int BC, bool MASK, int NK, bool VST>
__device__ __forceinline__ void s_phase(Smem<D, BC>& S, const half8_t (&qf)[D / 16], ScoreTile<NK / 32>& T,
                                        const Fetch<D, BC>* F, int64_t key0, int64_t qrow, int64_t Sk, int causal) {
  static_assert(NK % 32 == 0 && NK <= BC, "whole 32-key subtiles of the layout");
  const int lane = threadIdx.x & 63;
  const int hi = lane >> 5;  // which 16-key half of each 32-key group this lane holds
  constexpr int NG = NK / 32;
  constexpr int NS = D / 16;
  const half8_t* kbase = S.k + krow_of_lane(lane & 31) * Smem<D, BC>::KS8 + hi;
  auto mask_max = [&](int g) {
    if (MASK) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t key = key0 + 32 * g + 16 * hi + i;
        if (key >= Sk || (causal && key > qrow)) T.acc[g][i] = -__builtin_inff();
      }
    }
    T.bmax[g] = max16(T.acc[g]);
  };
  // Fragment reads run kAhead MFMAs ahead of their use (LDS latency is
  // several MFMA lengths) through a register ring; the fences keep reads and
  // MFMAs in this order and let only ALU work (the mask-and-max of the
  // previous subtile) move between them; the V staging words sit at fixed
  // iterations, spread over the loop.
  {
    constexpr int NM = NG * NS, kAhead = 4, kRing = kAhead + 2;
    constexpr int NW = Fetch<D, BC>::PER * 4;  // V staging words of this thread
    half8_t ring[kRing];
    auto kfrag = [&](int i) { return kbase[32 * (i / NS) * Smem<D, BC>::KS8 + 2 * (i % NS)]; };
#pragma unroll
    for (int i = 0; i < kAhead; ++i) ring[i] = kfrag(i);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int g = i / NS, s = i % NS;
      if (s == 0) T.acc[g] = float16_t{0};
      T.acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ring[i % kRing], qf[s], T.acc[g], 0, 0, 0);
      if (i + kAhead < NM) ring[(i + kAhead) % kRing] = kfrag(i + kAhead);
      if (s == 0 && g > 0) mask_max(g - 1);
      if (VST) {
#pragma unroll
        for (int q = 0; q < NW; ++q)
          if (i == (q * NM) / NW + 1) stage_v_word<D, BC>(*F, S, q / 4, q % 4);
      }
      __builtin_amdgcn_sched_barrier(0x0406);  // VALU, SALU and transcendental ops may cross (not MFMA, not LDS)
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  mask_max(NG - 1);
}

// Softmax, P and U^T += V^T P^T of a tile whose scores are in T.
template <int D, int BC, bool FP4, bool SINGLE, int NK>
__device__ __forceinline__ void pv_phase(const Smem<D, BC>& S, RowState<D>& R, ScoreTile<NK / 32>& T, float c) {
  const int lane = threadIdx.x & 63;
  const int hi = lane >> 5;
  constexpr int NG = NK / 32;
  float16_t (&acc)[NG] = T.acc;
  float (&bmax)[NG] = T.bmax;
  float smax = bmax[0];
#pragma unroll
  for (int g = 1; g < NG; ++g) smax = __builtin_fmaxf(smax, bmax[g]);
  smax = __builtin_fmaxf(smax, xor32(smax));
  const float tm = smax * c;  // tile row maximum of x = fl32(S c)
  // ---- reference update (rare after the first tiles)
  const bool live = tm > -__builtin_inff();
  const bool raise = live && tm > R.m + kRaise;
  if (__any(raise)) {
    const float f = raise ? __builtin_amdgcn_exp2f(R.m - tm) : 1.0f;  // R.m = -inf -> 0
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) R.o[t][i] = R.o[t][i] * f;
    R.l = R.l * f;
    if (raise) R.m = tm;
  }
  const bool use = live && tm >= R.m - kSkipBelow;
  if (!__any(use)) return;  // no row of this wave takes the tile
  // rows that skip the tile get offset -inf: every exponential below is 0
  const float ninf = -__builtin_inff();
  const half8_t* vbase = S.v + (lane & 31) * Smem<D, BC>::VS8 + hi;
  float lsum = 0.0f;
  // ---- P operands of subtile g, built in two halves (this lane's values
  // i = 8*h2 .. +8).  The subtile's level-2 scale data comes from the LDS
  // table (lookup, issued a subtile ahead of its use) and is then combined
  // with the row's offsets (finalize).
  struct PRaw {
    float lg, inv, s;
  };
  struct PPrep {
    float off, inv;
    half_t s2r;
  };
  auto lookup = [&](int g) {
    PRaw r{0.0f, 1.0f, 0.0f};
    if (FP4) {
      // level 2: s2 = E4M3(448 * max e) from the block maximum (single
      // level: s2 = E4M3(max e / 6))
      const float toff = use ? -tm : ninf;
      const float emax = __builtin_amdgcn_exp2f(__builtin_fmaf(bmax[g], c, toff));
      const uint32_t byte = f32_to_e4m3(SINGLE ? div6_rn(emax) : emax * 448.0f);
      const float4_t ps = S.pt[byte];
      r.lg = ps[0];
      r.inv = ps[1];
      r.s = ps[2];
    }
    return r;
  };
  // this row's weight of the tile relative to its reference, 2^(tm - m)
  const float rr = FP4 ? __builtin_amdgcn_exp2f(use ? tm - R.m : ninf) : 1.0f;
  auto finalize = [&](const PRaw& r) {
    PPrep q;
    if (FP4) {
      // the quantization inputs t = e * 2688 / s2 = 2^(x - tm + lg)
      q.off = use ? r.lg - tm : ninf;
      q.inv = r.inv;
      q.s2r = (half_t)(r.s * rr);
    } else {
      q.off = use ? -R.m : ninf;
      q.inv = 1.0f;
      q.s2r = (half_t)1.0f;
    }
    return q;
  };
  auto make_half = [&](int g, int h2, const PPrep& q, half8_t& pf) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[g][8 * h2 + i], c, q.off));
    float bsum = t[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) bsum += t[i];
    if (FP4) {
      // every byte of w is written below: its start value only lends the
      // register (t[0]'s, free once its pair is converted)
      uint32_t w = __float_as_uint(t[0]);
      w = cvt_pk_fp4<0>(w, t[0], t[1]);
      w = cvt_pk_fp4<1>(w, t[2], t[3]);
      w = cvt_pk_fp4<2>(w, t[4], t[5]);
      w = cvt_pk_fp4<3>(w, t[6], t[7]);
      pf = deq8(w, q.s2r);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) pf[i] = (half_t)t[i];
    }
    lsum = __builtin_fmaf(bsum, q.inv, lsum);
  };
  // ---- U^T += V^T P^T with V fragments through the same kind of ring; the P
  // halves of subtile g+1 are built between subtile g's MFMAs.
  {
    constexpr int NT = D / 32, NPV = 2 * NT, NM = NG * NPV, kAhead = 4, kRing = kAhead + 1;
    half8_t ring[kRing];
    // MFMA i: subtile g = i / NPV, h2 = (i % NPV) / NT, t = i % NT
    auto vfrag = [&](int i) {
      const int g = i / NPV, h2 = (i % NPV) / NT, t = i % NT;
      return vbase[Smem<D, BC>::vrow_t(t) + 4 * g + 2 * h2];
    };
#pragma unroll
    for (int i = 0; i < kAhead; ++i) ring[i] = vfrag(i);
    half8_t pcur[2], pnext[2];
    // the level-2 scale data of subtile g + 2 is looked up (an LDS read) a
    // whole subtile before its use, so that no wait drains the V ring
    PRaw rn = lookup(0);
    PPrep qn = finalize(rn);
    make_half(0, 0, qn, pcur[0]);
    make_half(0, 1, qn, pcur[1]);
    if (NG > 1) rn = lookup(1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int g = i / NPV, k = i % NPV, h2 = k / NT, t = k % NT;
      R.o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ring[i % kRing], pcur[h2], R.o[t], 0, 0, 0);
      if (i + kAhead < NM) ring[(i + kAhead) % kRing] = vfrag(i + kAhead);
      if (g + 1 < NG) {
        if (k == 1) {
          qn = finalize(rn);
          make_half(g + 1, 0, qn, pnext[0]);
          if (g + 2 < NG) rn = lookup(g + 2);
        }
        if (k == NPV / 2 + 1) make_half(g + 1, 1, qn, pnext[1]);
        if (k == NPV - 1) {
          pcur[0] = pnext[0];
          pcur[1] = pnext[1];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  // FP4: lsum is in units of e (tile-local); FP16: already in units of 2^m
  R.l += FP4 ? lsum * __builtin_amdgcn_exp2f(use ? tm - R.m : ninf) : lsum;
}

// Both phases of one tile (the FP16 path: its staging is done before).
template <int D, int BC, bool FP4, bool MASK, bool SINGLE, int NK = BC>
__device__ __forceinline__ void wave_tile(Smem<D, BC>& S, const half8_t (&qf)[D / 16], RowState<D>& R, int64_t key0,
                                          int64_t qrow, int64_t Sk, int causal, float c) {
  ScoreTile<NK / 32> T;
  s_phase<D, BC, MASK, NK, false>(S, qf, T, static_cast<const Fetch<D, BC>*>(nullptr), key0, qrow, Sk, causal);
  pv_phase<D, BC, FP4, SINGLE, NK>(S, R, T, c);
}

// One FP16-path step of ST keys at k0 (staged at the start of the tile
// layout) for this wave's rows [wrow0, wrow0 + 32).
template <int D, int BC, int ST>
__device__ __forceinline__ void fp16_step(Smem<D, BC>& S, const half8_t (&qf)[D / 16], RowState<D>& R,
                                          int64_t k0, int64_t wrow0, int64_t qrow, int64_t Sk, int causal, float c) {
  if (causal && k0 > wrow0 + 31) return;  // every key after this wave's rows
  const bool need_mask = (k0 + ST > Sk) || (causal && k0 + ST - 1 > wrow0);
  if (need_mask) wave_tile<D, BC, false, true, false, ST>(S, qf, R, k0, qrow, Sk, causal, c);
  else wave_tile<D, BC, false, false, false, ST>(S, qf, R, k0, qrow, Sk, causal, c);
}

// The selection list of a query block, read 64 entries at a time into one
// register (lane i holds entry base + i) and looked up with readlane: the tile
// loops make no memory access and no wait for it.  Entries past the count n
// read as INT32_MAX (above every block index).
struct SelList {
  const int32_t* sel;
  int n, cap, base, chunk;  // n: entries in use; cap: entries the list holds (reads stay below it)
  __device__ __forceinline__ void init(const int32_t* s, int capacity) {
    sel = s;
    n = capacity;
    cap = capacity;
    base = 0;
    chunk = fetch(0);
  }
  __device__ __forceinline__ int fetch(int b) const {
    const int i = b + (int)(threadIdx.x & 63);
    return i < cap ? sel[i] : 0x7fffffff;
  }
  // entry i (wave-uniform), INT32_MAX past the count
  __device__ __forceinline__ int get(int i) {
    if (i >= n) return 0x7fffffff;
    if (i < base || i >= base + 64) {
      base = i & ~63;
      chunk = fetch(base);
    }
    return __builtin_amdgcn_readlane(chunk, i - base);
  }
};

// The FP16 pass's walk over the selected blocks: steps of STEP keys in list
// order.  An entry not above every earlier entry is skipped (negative ones
// included); once a block starts at or past kend the walk ends, since every
// later entry that is not skipped lies further out.
template <int STEP>
struct SelCursor {
  SelList* list;
  int halves, sel_block;  // halves: steps per block
  int64_t kend;
  int s_i = -1, hh = 0, prev = -1;
  int64_t base = 0;
  // key0 of the next step, or -1
  __device__ __forceinline__ int64_t next() {
    const int nsel = list->n;
    if (s_i >= 0 && s_i < nsel) {
      ++hh;
      if (hh < halves && base + (int64_t)STEP * hh < kend) return base + (int64_t)STEP * hh;
    }
    int v = 0;
    while (++s_i < nsel && (v = list->get(s_i)) <= prev) {
    }
    if (s_i >= nsel) return -1;
    prev = v;
    hh = 0;
    base = (int64_t)prev * sel_block;
    if (base >= kend) {
      s_i = nsel;
      return -1;
    }
    return base;
  }
};

// PM: P on the FP4 tiles -- 0 two-level, 1 single-level, 2 unquantized
// (fp16 probabilities with the FP4 operands: the high-precision output O' of
// training, Attn-QAT page, Metodologia / A).
// STR: q, k, v rows through their row maps (strided inputs; only the FP16
// path reads them), else dense.
template <int D, int BC, typename IT, typename OT, int PM, bool STR>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(Problem P) {
  __shared__ Smem<D, BC> S;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hi = lane >> 5;
  // workgroup -> (batch*head, query tile).  Workgroups go round-robin to the 8
  // XCDs.  With P.xcd_heads each XCD takes whole heads, one after the other,
  // so the workgroups resident on an XCD stream the same K/V (and the same
  // promoted bf16 tiles) through its L2, the heaviest (causal) query tiles of
  // a head first.  Otherwise heads are interleaved over the XCDs and the
  // heaviest query tiles of all heads come first.
  const int64_t BH = gridDim.x / P.nqt;
  int64_t bh, qrank;
  const int64_t gi = blockIdx.x;
  if (P.xcd_heads && BH % 8 == 0) {
    const int64_t xcd = gi % 8, slot = gi / 8;
    qrank = slot % P.nqt;
    bh = (slot / P.nqt) * 8 + xcd;
  } else {
    bh = gi % BH;
    qrank = gi / BH;
  }
  const int qt = (int)(P.causal ? (P.nqt - 1 - qrank) : qrank);
  const int64_t b = bh / P.H, h = bh - b * P.H, hk = h / (P.H / P.Hkv);
  const int64_t q0 = (int64_t)qt * kBr;
  const int64_t qrow = q0 + 32 * wave + (lane & 31);
  const int64_t Sk = P.Sk;

  // selection of this query block (sel_block is a multiple of kBr); its list
  // and count load while the Q fragment below does
  const int32_t* sel = nullptr;
  int nsel = 0;
  SelList list;
  if (P.pct > 0) {
    const int64_t qb = q0 / P.sel_block;
    sel = P.idx + (bh * P.nqb + qb) * P.kmax;
    nsel = P.cnt[bh * P.nqb + qb];
    list.init(sel, P.kmax);
    nsel = nsel < 0 ? 0 : (nsel > P.kmax ? P.kmax : nsel);  // a given count never reaches the padding
  } else {
    list.init(nullptr, 0);
  }
  list.n = nsel;
  const float4_t ptv = PM == 1 ? kPScale1.v[threadIdx.x & 127] : kPScale.v[threadIdx.x & 127];
  // Q^ fragment (B operand): query qrow, d = 16 s + 8 hi .. +8
  half8_t qf[D / 16];
  {
    // rows past Sq read row 0 (every load in bounds and in flight together)
    // and are zeroed
    const bool ok = qrow < P.Sq;
    const uint8_t* qcr = P.qc + (bh * P.Sq + (ok ? qrow : 0)) * (D / 2);
    const uint8_t* qsr = P.qs + (bh * P.Sq + (ok ? qrow : 0)) * (D / 16);
    uint32_t cws[D / 16];
    uint8_t scs[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      cws[s] = *reinterpret_cast<const uint32_t*>(qcr + 8 * s + 4 * hi);
      scs[s] = qsr[s];
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint32_t cw = ok ? cws[s] : 0u;
      const half_t sc = (half_t)e4m3_to_f32(ok ? scs[s] : 0u);
      half2_t a = scale_pair(cvt_pk_f16_fp4<0>(cw), sc), bb = scale_pair(cvt_pk_f16_fp4<1>(cw), sc);
      half2_t cc = scale_pair(cvt_pk_f16_fp4<2>(cw), sc), dd = scale_pair(cvt_pk_f16_fp4<3>(cw), sc);
      qf[s] = half8_t{a[0], a[1], bb[0], bb[1], cc[0], cc[1], dd[0], dd[1]};
    }
  }
  // level-2 P scale table (read after the first barrier of the tile loop)
  if (threadIdx.x < 128) S.pt[threadIdx.x] = ptv;
  RowState<D> R;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) R.o[t] = float16_t{0};
  R.m = -__builtin_inff();
  R.l = 0.0f;

  const int64_t qend = q0 + kBr < P.Sq ? q0 + kBr : P.Sq;  // rows of this workgroup: [q0, qend)
  int64_t kend = Sk;
  if (P.causal && qend < kend) kend = qend;
  const int ntile = (int)((kend + BC - 1) / BC);
  const int tiles_per_block = P.sel_block / BC;

  const int64_t bhk = b * P.Hkv + hk;
  HeadBufs hb;
  hb.kc = make_rsrc(P.kc + bhk * Sk * (D / 2), (uint32_t)(Sk * (D / 2)));
  hb.ks = make_rsrc(P.ks + bhk * Sk * (D / 16), (uint32_t)(Sk * (D / 16)));
  hb.vc = make_rsrc(P.vc + bhk * (Sk / 2) * D, (uint32_t)((Sk / 2) * D));
  hb.vs = make_rsrc(P.vs + bhk * (Sk / 16) * D, (uint32_t)((Sk / 16) * D));

  // ---- FP4 pass: every tile not covered by a selected block.  A block
  // counts as selected when its index exceeds every list entry before it (the
  // whole list, for the ascending lists the selection kernel writes); the FP16
  // pass below takes exactly these entries, so a given list that is unsorted
  // or repeats an index never counts a key twice or skips it.
  Fetch<D, BC> F;
  int si = 0, sv = list.get(0);  // cursor into the selection list and its entry
  auto selected = [&](int tile) {
    if (nsel == 0) return false;
    const int blk = tile / tiles_per_block;
    while (sv < blk) sv = list.get(++si);
    return sv == blk;
  };
  int cur = 0;
  while (cur < ntile && selected(cur)) ++cur;
  if (cur < ntile) {
    fetch_k<D, BC>(F, hb, (int64_t)cur * BC);
    fetch_v<D, BC>(F, hb, (int64_t)cur * BC);
  }
  // per tile: K staged between the first two barriers, V between the scores'
  // MFMAs (a wave with no visible key in the tile stages its V share alone),
  // and the third barrier before any wave reads V.  Every barrier is reached
  // by every wave.
  while (cur < ntile) {
    int nxt = cur + 1;
    while (nxt < ntile && selected(nxt)) ++nxt;
    // always prefetch (past the last tile this is a harmless cached reload)
    const int64_t knext = (int64_t)(nxt < ntile ? nxt : cur) * BC;
    __syncthreads();  // previous tile's LDS reads are done
    stage_k<D, BC>(F, S);
    fetch_k<D, BC>(F, hb, knext);
    __syncthreads();
    const int64_t key0 = (int64_t)cur * BC;
    const int64_t wrow0 = q0 + 32 * wave;
    const bool wave_dead = P.causal && key0 > wrow0 + 31;  // every key of the tile is after this wave's rows
    ScoreTile<BC / 32> T;
    if (!wave_dead) {
      const bool need_mask = (key0 + BC > Sk) || (P.causal && key0 + BC - 1 > wrow0);
      if (need_mask) s_phase<D, BC, true, BC, true>(S, qf, T, &F, key0, qrow, Sk, P.causal);
      else s_phase<D, BC, false, BC, true>(S, qf, T, &F, key0, qrow, Sk, P.causal);
    } else {
      stage_v<D, BC>(F, S);
    }
    fetch_v<D, BC>(F, hb, knext);
    __syncthreads();  // V is staged
    if (!wave_dead) pv_phase<D, BC, PM != 2, PM == 1, BC>(S, R, T, P.c);
    cur = nxt;
  }

  // FP4 tiles accumulated P^ V^ with P^ in units of e/2688 (two-level) or of e
  const float to_e = PM == 0 ? 1.0f / 2688.0f : 1.0f;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) R.o[t][i] = R.o[t][i] * to_e;

  // ---- FP16 pass over the selected blocks
  if (nsel > 0) {
    // fp16 Q fragment from the original input
    const IT* qp = reinterpret_cast<const IT*>(P.q) + (STR ? P.qmap.head_off(bh) : bh * P.Sq * D);
    const int64_t qts = STR ? P.qmap.ts : D;
    const bool ok = qrow < P.Sq;
    uint4_t qw[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qw[s] = *reinterpret_cast<const uint4_t*>(qp + (ok ? qrow : 0) * qts + 16 * s + 8 * hi);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      uint4_t w = ok ? qw[s] : uint4_t{0, 0, 0, 0};
      half2_t a = to_half2<IT>(w[0]), bb = to_half2<IT>(w[1]), cc = to_half2<IT>(w[2]), dd = to_half2<IT>(w[3]);
      qf[s] = half8_t{a[0], a[1], bb[0], bb[1], cc[0], cc[1], dd[0], dd[1]};
    }
    // one head's token rows (the host checks that (Sk - 1) ts + D elements fit 32-bit byte offsets)
    const uint32_t kts = STR ? (uint32_t)P.kmap.ts : D, vts = STR ? (uint32_t)P.vmap.ts : D;
    const rsrc_t kr16 = make_rsrc(reinterpret_cast<const IT*>(P.k) + (STR ? P.kmap.head_off(bhk) : bhk * Sk * D),
                                  (uint32_t)(((Sk - 1) * kts + D) * 2));
    const rsrc_t vr16 = make_rsrc(reinterpret_cast<const IT*>(P.v) + (STR ? P.vmap.head_off(bhk) : bhk * Sk * D),
                                  (uint32_t)(((Sk - 1) * vts + D) * 2));
    // steps of the selected blocks in list order, each fetched into
    // registers while the step before it computes
    constexpr int ST = kStepKeys<D>;
    SelCursor<ST> cur{&list, P.sel_block / ST, P.sel_block, kend};
    const int64_t wrow0 = q0 + 32 * wave;
    Fetch16<D> G;
    int64_t key0 = cur.next();
    if (key0 >= 0) fetch16<D>(G, kr16, vr16, kts, vts, key0);
    while (key0 >= 0) {
      const int64_t nxt = cur.next();
      __syncthreads();  // previous step's LDS reads are done
      stage16<D, BC, IT>(G, S);
      if (nxt >= 0) fetch16<D>(G, kr16, vr16, kts, vts, nxt);
      __syncthreads();
      fp16_step<D, BC, ST>(S, qf, R, key0, wrow0, qrow, Sk, P.causal, P.c);
      key0 = nxt;
    }
  }

  // ---- epilogue: O / l, lse
  const float ltot = R.l + xor32(R.l);
  if (qrow < P.Sq) {
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    OT* orow = reinterpret_cast<OT*>(P.out) + (bh * P.Sq + qrow) * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * t + 8 * j + 4 * hi;
        store4<OT>(orow + d0, R.o[t][4 * j] * inv, R.o[t][4 * j + 1] * inv, R.o[t][4 * j + 2] * inv,
                   R.o[t][4 * j + 3] * inv);
      }
    if (P.lse && hi == 0)
      P.lse[bh * P.Sq + qrow] = ltot > 0.0f ? (R.m + __builtin_log2f(ltot)) * 0.69314718055994531f : -__builtin_inff();
  }
}

template <int D, int BC, typename IT, int PM, bool STR>
hipError_t launch_str(const AttnLaunch& L, const Problem& P, dim3 grid, hipStream_t st) {
  if (L.out_dtype == 2) hipLaunchKernelGGL((attn_fwd_kernel<D, BC, IT, float, PM, STR>), grid, dim3(256), 0, st, P);
  else if (L.out_dtype == 1) hipLaunchKernelGGL((attn_fwd_kernel<D, BC, IT, half_t, PM, STR>), grid, dim3(256), 0, st, P);
  else hipLaunchKernelGGL((attn_fwd_kernel<D, BC, IT, uint16_t, PM, STR>), grid, dim3(256), 0, st, P);
  return hipGetLastError();
}

// The strided instances only where the FP16 path runs (a budget; P modes 0
// and 1): without it the kernel reads only the quantized operands.
template <int D, int BC, typename IT, int PM>
hipError_t launch_out(const AttnLaunch& L, const Problem& P, dim3 grid, hipStream_t st) {
  if constexpr (PM != 2) {
    if (L.strided && L.pct > 0) return launch_str<D, BC, IT, PM, true>(L, P, grid, st);
  }
  return launch_str<D, BC, IT, PM, false>(L, P, grid, st);
}

template <int D, int BC>
hipError_t launch_in(const AttnLaunch& L, const Problem& P, dim3 grid, hipStream_t st) {
  // P mode x input type x output type
  if (L.p_mode == 1) {
    if (L.dtype == 1) return launch_out<D, BC, half_t, 1>(L, P, grid, st);
    return launch_out<D, BC, uint16_t, 1>(L, P, grid, st);
  }
  if (L.p_mode == 2) {
    if (L.dtype == 1) return launch_out<D, BC, half_t, 2>(L, P, grid, st);
    return launch_out<D, BC, uint16_t, 2>(L, P, grid, st);
  }
  if (L.dtype == 1) return launch_out<D, BC, half_t, 0>(L, P, grid, st);
  return launch_out<D, BC, uint16_t, 0>(L, P, grid, st);
}

}  // namespace fp4dev

using namespace fp4dev;

hipError_t fp4i_launch_attn_fwd(const AttnLaunch& L, hipStream_t st) {
  Problem P;
  P.H = L.H; P.Hkv = L.Hkv; P.Sq = L.Sq; P.Sk = L.Sk;
  P.qc = L.qc; P.qs = L.qs; P.kc = L.kc; P.ks = L.ks; P.vc = L.vc; P.vs = L.vs;
  P.q = L.q; P.k = L.k; P.v = L.v;
  P.qmap = L.qmap; P.kmap = L.kmap; P.vmap = L.vmap;
  P.idx = L.idx; P.cnt = L.cnt;
  P.causal = L.causal; P.pct = L.pct; P.sel_block = L.pct > 0 ? L.sel_block : 128;
  P.nqb = L.nqb; P.kmax = L.kmax;
  P.c = L.c;
  P.out = L.out; P.lse = L.lse;
  P.nqt = (int)((L.Sq + kBr - 1) / kBr);
  // Whole heads per XCD pay off where a budget's promoted bf16 tiles are
  // re-read from L2 by the head's other query blocks and a head's bf16 K/V
  // (Sk d 4 bytes) exceeds two L2s; elsewhere interleaved heads, heaviest
  // tiles first over all heads, balance better.  Measured (32 heads, d 128,
  // causal): interleaved 21-25% faster at 4K, 1-2% at 8K and 16K, the same at
  // 32K without a budget, 4.7% slower at 32K with a 10% budget.
  P.xcd_heads = L.pct > 0 && L.Sk * L.d * 4 > ((int64_t)8 << 20) ? 1 : 0;
  dim3 grid((unsigned)(L.B * L.H * P.nqt));
  if (L.d == 128) {
    if (L.kv_tile == 128) return launch_in<128, 128>(L, P, grid, st);
    return launch_in<128, 64>(L, P, grid, st);
  }
  if (L.kv_tile == 128) return launch_in<64, 128>(L, P, grid, st);
  return launch_in<64, 64>(L, P, grid, st);
}

// attn_mx.hip -- MXFP4 variant of the fused attention forward, on gfx950's
// block-scaled FP4 matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4.
//
// Operands are MXFP4: E2M1 codes with one power-of-two (E8M0) scale per 32
// elements -- Q and K blocked along d, V along tokens, P along keys -- the
// classic block floating point the ScaleSearch page contrasts NVFP4 with
// (Declaracion del Problema).  The instruction takes those scales directly,
// so nothing is dequantized: the codes go from HBM to LDS as they are and
// the matrix core runs at its FP4 rate (four times the fp16 rate).
//
// What it computes, per query row i and key tile T of kv_tile keys:
//   x = fl32(S c), S = Q^ K^T;  tm = max over visible keys;  the tile
//   reference is ceil(tm) (a power of two, so it can ride on the E8M0 scale);
//   e = 2^(x - ceil(tm));  per 32 keys, P^ = MXFP4(e) (scale 2^(floor(log2
//   max e) - 2), codes RNE_E2M1(e / scale)); the tile adds P^ V^ with weight
//   2^(ceil(tm) - m) folded into P^'s scale byte; l sums the unquantized e.
//
// MI355X mapping (4 waves x 32 query rows per workgroup, as the NVFP4 kernel):
//   - S^T = K^ Q^T: A = 32 keys x 64 d of K codes from LDS (rows fed in the
//     permuted order that leaves each lane 16 consecutive keys of its query),
//     B = the wave's Q codes in registers, scale bytes per (row, 32 d);
//   - the lane pair (l, l^32) holds a query's 32-key block: the block maximum
//     crosses once, the lane quantizes its 16 keys, and one permlane32 swap
//     turns two subtiles' codes into the P^T operand (32 consecutive keys per
//     lane) of O^T += V^T P^T, with V^T codes staged transposed in LDS by 4x4
//     byte transposes;
//   - the running reference m is integer, so every rescale is exact.
#include "device_common.h"
#include "fp4_internal.h"

namespace fp4dev {
namespace mxattn {

constexpr int kWaves = 4;
constexpr int kBr = 32 * kWaves;
constexpr float kRaise = 8.0f;       // the reference moves when a tile exceeds it by more than 2^8
constexpr float kSkipBelow = 64.0f;  // tiles more than 2^64 below the reference are left out

typedef int v8i_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// A-operand row of S^T for key k of a 32-key subtile: output row r holds key
// krow(r) = (r%4) + 4(r/8) + 16((r/4)%2), so lane (query, hi) ends up with
// keys 16 hi .. 16 hi + 15 of the subtile.
__device__ __forceinline__ int krow_of_lane(int r) { return (r & 3) | ((r >> 3) << 2) | (((r >> 2) & 1) << 4); }

__device__ __forceinline__ float16_t mfma_fp4(uint4_t a, uint4_t b, float16_t c, uint32_t sa, uint32_t sb) {
  const v8i_t av = v8i_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const v8i_t bv = v8i_t{(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// LDS tile: K codes [key][D/2] and V^T codes [channel][BC/2] with one 16-byte
// unit of padding per row (a half-wave's 16-byte reads of 32 rows then fall
// on distinct bank groups), K scales [key][D/32], V scales [BC/32][D].
template <int D, int BC>
struct MxSmem {
  static constexpr int KROW = D / 2 + 16;
  static constexpr int VROW = BC / 2 + 16;
  uint8_t k[BC * KROW];
  uint8_t v[D * VROW];
  uint8_t ks[BC * (D / 32)];
  uint8_t vs[(BC / 32) * D];
};

// One tile's raw codes and scales in registers between fetch and stage.
// K: chunk u covers 16 bytes of key row (id / (D/32)); V: a 4 x 4 byte block
// (4 token pairs x 4 channels) per task.
template <int D, int BC>
struct MxFetch {
  static constexpr int KCH = BC * D / 32;        // 16-byte K chunks per tile
  static constexpr int KPER = (KCH + 255) / 256; // per thread
  static constexpr int VT = (BC / 8) * (D / 4);  // 4x4 byte blocks per tile
  static constexpr int VPER = (VT + 255) / 256;
  static constexpr int KSB = BC * (D / 32);      // K scale bytes
  static constexpr int VSB = (BC / 32) * D;      // V scale bytes
  uint4_t kc[KPER];
  uint32_t vc[VPER][4];
  uint32_t ks, vs;  // 4 scale bytes each (threads below KSB/4, VSB/4)
};

struct MxProblem {
  int64_t H, Hkv, Sq, Sk;
  const uint8_t *qc, *qs, *kc, *ks, *vc, *vs;
  int causal, nqt;
  float c;
  void* out;
  float* lse;
};

struct MxHead {
  rsrc_t kc, ks, vc, vs;
};

template <int D, int BC>
__device__ __forceinline__ void mx_fetch(MxFetch<D, BC>& F, const MxHead& hb, int64_t key0) {
  using Fe = MxFetch<D, BC>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < Fe::KPER; ++u) {
    const int id = tid + 256 * u;
    if (Fe::KCH % 256 && id >= Fe::KCH) break;
    const uint32_t row = (uint32_t)key0 + id / (D / 32), cu = id % (D / 32);
    F.kc[u] = buf_load16(hb.kc, row * (D / 2) + cu * 16);
  }
#pragma unroll
  for (int u = 0; u < Fe::VPER; ++u) {
    const int id = tid + 256 * u;
    if (Fe::VT % 256 && id >= Fe::VT) break;
    const int pg = id / (D / 4), cg = id % (D / 4);
    const uint32_t pair0 = (uint32_t)(key0 / 2) + 4 * pg;
#pragma unroll
    for (int i = 0; i < 4; ++i) F.vc[u][i] = buf_load4(hb.vc, (pair0 + i) * D + 4 * cg);
  }
  if (tid < Fe::KSB / 4) F.ks = buf_load4(hb.ks, (uint32_t)key0 * (D / 32) + 4 * tid);
  if (tid < Fe::VSB / 4) F.vs = buf_load4(hb.vs, (uint32_t)(key0 / 32) * D + 4 * tid);
}

// 4x4 byte transpose: o[j] = byte j of a, b, c, d (in that order).
__device__ __forceinline__ void transpose4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t* o) {
  const uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  const uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u);
  const uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);  // a0 b0 c0 d0
  o[1] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);  // a1 b1 c1 d1
  o[2] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);
}

template <int D, int BC>
__device__ __forceinline__ void mx_stage(const MxFetch<D, BC>& F, MxSmem<D, BC>& S) {
  using Fe = MxFetch<D, BC>;
  using Sm = MxSmem<D, BC>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < Fe::KPER; ++u) {
    const int id = tid + 256 * u;
    if (Fe::KCH % 256 && id >= Fe::KCH) break;
    const int row = id / (D / 32), cu = id % (D / 32);
    *reinterpret_cast<uint4_t*>(S.k + row * Sm::KROW + cu * 16) = F.kc[u];
  }
#pragma unroll
  for (int u = 0; u < Fe::VPER; ++u) {
    const int id = tid + 256 * u;
    if (Fe::VT % 256 && id >= Fe::VT) break;
    const int pg = id / (D / 4), cg = id % (D / 4);
    uint32_t o[4];
    transpose4(F.vc[u][0], F.vc[u][1], F.vc[u][2], F.vc[u][3], o);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(S.v + (4 * cg + j) * Sm::VROW + 4 * pg) = o[j];
  }
  if (tid < Fe::KSB / 4) *reinterpret_cast<uint32_t*>(S.ks + 4 * tid) = F.ks;
  if (tid < Fe::VSB / 4) *reinterpret_cast<uint32_t*>(S.vs + 4 * tid) = F.vs;
}

template <int D>
struct MxRow {
  float16_t o[D / 32];  // O^T: channels 32 t + (v%4) + 8 (v/4) + 4 hi, query lane%32
  float m;              // integer reference exponent (x units), -inf before the first tile
  float l;              // this lane's part of the denominator, in units of 2^m
};

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

template <int D, int BC, bool MASK>
__device__ __forceinline__ void mx_wave_tile(const MxSmem<D, BC>& S, const uint4_t (&qf)[D / 64],
                                             const uint32_t (&qsc)[D / 64], MxRow<D>& R, int64_t key0, int64_t qrow,
                                             int64_t Sk, int causal, float c) {
  using Sm = MxSmem<D, BC>;
  constexpr int NG = BC / 32, NC = D / 64, NT = D / 32;
  const int lane = threadIdx.x & 63, hi = lane >> 5, r32 = lane & 31;
  // ---- S^T = K^ Q^T
  float16_t acc[NG];
  const int krow = krow_of_lane(r32);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int row = 32 * g + krow;
    const uint32_t ksw = D == 128 ? *reinterpret_cast<const uint32_t*>(S.ks + row * (D / 32))
                                  : (uint32_t)*reinterpret_cast<const uint16_t*>(S.ks + row * (D / 32));
    acc[g] = float16_t{0};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const uint4_t a = *reinterpret_cast<const uint4_t*>(S.k + row * Sm::KROW + 32 * cc + 16 * hi);
      acc[g] = mfma_fp4(a, qf[cc], acc[g], (ksw >> (8 * (2 * cc + hi))) & 0xFFu, qsc[cc]);
    }
  }
  float bmax[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (MASK) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t key = key0 + 32 * g + 16 * hi + i;
        if (key >= Sk || (causal && key > qrow)) acc[g][i] = -__builtin_inff();
      }
    }
    bmax[g] = max16(acc[g]);
  }
  float smax = bmax[0];
#pragma unroll
  for (int g = 1; g < NG; ++g) smax = __builtin_fmaxf(smax, bmax[g]);
  smax = __builtin_fmaxf(smax, xor32(smax));
  const float tm = smax * c;
  const bool live = tm > -__builtin_inff();
  const float tmc = live ? __builtin_ceilf(tm) : -__builtin_inff();
  // ---- reference update (integer steps: exact rescale)
  const bool raise = live && tmc > R.m + kRaise;
  if (__any(raise)) {
    const float f = raise ? __builtin_amdgcn_exp2f(R.m - tmc) : 1.0f;  // R.m = -inf -> 0
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) R.o[t][i] = R.o[t][i] * f;
    R.l = R.l * f;
    if (raise) R.m = tmc;
  }
  const bool use = live && tmc >= R.m - kSkipBelow;
  if (!__any(use)) return;
  const float off = use ? -tmc : -__builtin_inff();
  const int rexp = use ? (int)(tmc - R.m) : 0;  // the tile's weight 2^rexp, -64 <= rexp <= 8
  // ---- P^: per 32-key block (this lane's 16 keys and its partner's 16)
  uint32_t pc[NG][2];
  uint32_t psb[NG];
  float lsum = 0.0f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float em = __builtin_amdgcn_exp2f(__builtin_fmaf(bmax[g], c, off));
    em = __builtin_fmaxf(em, xor32(em));
    int sh = em > 0.0f ? __builtin_amdgcn_frexp_expf(em) - 3 : -127;  // floor(log2 max e) - 2
    sh = sh < -127 ? -127 : sh;
    // the quantization inputs t = e / 2^sh come out of one exp2: the reference and the shift
    // are integers, so off - sh is exact; the denominator takes the block sum of t times 2^sh
    const float offs = off - (float)sh;
    float t[16], bs = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      t[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[g][i], c, offs));
      bs += t[i];
    }
    lsum += __builtin_ldexpf(bs, sh);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w = 0;
      w = cvt_pk_fp4<0>(w, t[8 * h + 0], t[8 * h + 1]);
      w = cvt_pk_fp4<1>(w, t[8 * h + 2], t[8 * h + 3]);
      w = cvt_pk_fp4<2>(w, t[8 * h + 4], t[8 * h + 5]);
      w = cvt_pk_fp4<3>(w, t[8 * h + 6], t[8 * h + 7]);
      pc[g][h] = w;
    }
    int sb = sh + 127 + rexp;  // the tile weight rides on the block scale
    psb[g] = (uint32_t)(sb < 0 ? 0 : sb);
  }
  R.l += __builtin_ldexpf(lsum, rexp);
  // ---- O^T += V^T P^T, 64 keys per instruction
#pragma unroll
  for (int kc = 0; kc < BC / 64; ++kc) {
    const auto w0 = __builtin_amdgcn_permlane32_swap(pc[2 * kc][0], pc[2 * kc + 1][0], false, false);
    const auto w1 = __builtin_amdgcn_permlane32_swap(pc[2 * kc][1], pc[2 * kc + 1][1], false, false);
    const uint4_t b = uint4_t{w0[0], w1[0], w0[1], w1[1]};
    const uint32_t sbb = hi ? psb[2 * kc + 1] : psb[2 * kc];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int ch = 32 * t + r32;
      const uint4_t a = *reinterpret_cast<const uint4_t*>(S.v + ch * Sm::VROW + 32 * kc + 16 * hi);
      const uint32_t sa = S.vs[(2 * kc + hi) * D + ch];
      R.o[t] = mfma_fp4(a, b, R.o[t], sa, sbb);
    }
  }
}

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
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  uint2_t w;
  w[0] = (uint32_t)to_bf16(a) | ((uint32_t)to_bf16(b) << 16);
  w[1] = (uint32_t)to_bf16(c) | ((uint32_t)to_bf16(d) << 16);
  *reinterpret_cast<uint2_t*>(p) = w;
}

template <int D, int BC, typename OT>
__global__ void __launch_bounds__(256, 2) mx_attn_kernel(MxProblem P) {
  __shared__ MxSmem<D, BC> S;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hi = lane >> 5;
  // workgroup -> (batch*head, query tile).  Workgroups go round-robin to the
  // 8 XCDs.  Where a head's K and V codes fill an L2 (Sk d >= 4 Mi bytes), each
  // XCD takes whole heads, one after the other (their codes stay in its L2),
  // the heaviest causal tiles of a head first; below that, heads are
  // interleaved over the XCDs and the heaviest tiles of all heads come first
  // (measured at 32 heads, d 128, causal: 8K 10-12% faster interleaved, 32K
  // up to 2.5% faster with whole heads).
  const int64_t BH = gridDim.x / P.nqt;
  int64_t bh, qrank;
  const int64_t gi = blockIdx.x;
  if (BH % 8 == 0 && P.Sk * D >= ((int64_t)4 << 20)) {
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
  // Q codes and scales (B operand): query qrow, d = 64 cc + 32 hi .. +32
  uint4_t qf[D / 64];
  uint32_t qsc[D / 64];
  {
    const bool ok = qrow < P.Sq;
    const uint8_t* qcr = P.qc + (bh * P.Sq + (ok ? qrow : 0)) * (D / 2);
    const uint8_t* qsr = P.qs + (bh * P.Sq + (ok ? qrow : 0)) * (D / 32);
#pragma unroll
    for (int cc = 0; cc < D / 64; ++cc) {
      qf[cc] = ok ? *reinterpret_cast<const uint4_t*>(qcr + 32 * cc + 16 * hi) : uint4_t{0, 0, 0, 0};
      qsc[cc] = ok ? (uint32_t)qsr[2 * cc + hi] : 0u;
    }
  }
  MxRow<D> R;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) R.o[t] = float16_t{0};
  R.m = -__builtin_inff();
  R.l = 0.0f;
  const int64_t qend = q0 + kBr < P.Sq ? q0 + kBr : P.Sq;
  int64_t kend = Sk;
  if (P.causal && qend < kend) kend = qend;
  const int ntile = (int)((kend + BC - 1) / BC);
  const int64_t bhk = b * P.Hkv + hk;
  MxHead hb;
  hb.kc = make_rsrc(P.kc + bhk * Sk * (D / 2), (uint32_t)(Sk * (D / 2)));
  hb.ks = make_rsrc(P.ks + bhk * Sk * (D / 32), (uint32_t)(Sk * (D / 32)));
  hb.vc = make_rsrc(P.vc + bhk * (Sk / 2) * D, (uint32_t)((Sk / 2) * D));
  hb.vs = make_rsrc(P.vs + bhk * (Sk / 32) * D, (uint32_t)((Sk / 32) * D));
  MxFetch<D, BC> F;
  if (ntile > 0) mx_fetch<D, BC>(F, hb, 0);
  for (int cur = 0; cur < ntile; ++cur) {
    __syncthreads();  // the previous tile's LDS reads are done
    mx_stage<D, BC>(F, S);
    if (cur + 1 < ntile) mx_fetch<D, BC>(F, hb, (int64_t)(cur + 1) * BC);
    __syncthreads();
    const int64_t key0 = (int64_t)cur * BC;
    const int64_t wrow0 = q0 + 32 * wave;
    const bool wave_dead = P.causal && key0 > wrow0 + 31;
    if (!wave_dead) {
      const bool need_mask = (key0 + BC > Sk) || (P.causal && key0 + BC - 1 > wrow0);
      if (need_mask) mx_wave_tile<D, BC, true>(S, qf, qsc, R, key0, qrow, Sk, P.causal, P.c);
      else mx_wave_tile<D, BC, false>(S, qf, qsc, R, key0, qrow, Sk, P.causal, P.c);
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

template <int D, int BC>
hipError_t launch_mx(const MxAttnLaunch& L, const MxProblem& P, dim3 grid, hipStream_t st) {
  if (L.out_dtype == 2) hipLaunchKernelGGL((mx_attn_kernel<D, BC, float>), grid, dim3(256), 0, st, P);
  else if (L.out_dtype == 1) hipLaunchKernelGGL((mx_attn_kernel<D, BC, half_t>), grid, dim3(256), 0, st, P);
  else hipLaunchKernelGGL((mx_attn_kernel<D, BC, uint16_t>), grid, dim3(256), 0, st, P);
  return hipGetLastError();
}

}  // namespace mxattn
}  // namespace fp4dev

using namespace fp4dev;

hipError_t fp4i_launch_attn_mx(const MxAttnLaunch& L, hipStream_t st) {
  mxattn::MxProblem P;
  P.H = L.H; P.Hkv = L.Hkv; P.Sq = L.Sq; P.Sk = L.Sk;
  P.qc = L.qc; P.qs = L.qs; P.kc = L.kc; P.ks = L.ks; P.vc = L.vc; P.vs = L.vs;
  P.causal = L.causal;
  P.c = L.c;
  P.out = L.out;
  P.lse = L.lse;
  P.nqt = (int)((L.Sq + mxattn::kBr - 1) / mxattn::kBr);
  const dim3 grid((unsigned)(L.B * L.H * P.nqt));
  if (L.d == 128) {
    if (L.kv_tile == 128) return mxattn::launch_mx<128, 128>(L, P, grid, st);
    return mxattn::launch_mx<128, 64>(L, P, grid, st);
  }
  if (L.kv_tile == 128) return mxattn::launch_mx<64, 128>(L, P, grid, st);
  return mxattn::launch_mx<64, 64>(L, P, grid, st);
}

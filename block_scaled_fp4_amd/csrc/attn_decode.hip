// attn_decode.hip -- one-token decode over a sink-aware mixed-precision KV
// cache (ScaleSearch page, Metodologia / ScaleSearchAttention: the first and
// last cache blocks stay in full precision, the rest in NVFP4).
//
// Decode is bound by HBM: every cached byte is read once per step and used by
// only the G = Hq/Hkv query heads of its group.  MI355X mapping:
//   - the FP4 region of every (batch, kv head) is split into many chunks of
//     split_len tokens, one workgroup each, so a 16 x 8 batch-head grid still
//     puts thousands of workgroups on 256 CUs; one extra split per (batch, kv
//     head) reads the bf16 sink and recent tokens;
//   - a workgroup streams 128-key tiles: all 256 lanes fetch the next tile's
//     codes into registers while the current tile computes, and dequantize
//     into LDS (K as [key][d], V transposed as [d][key], both fp16: exact);
//   - each wave owns 32 keys of the tile: S^T = K q^T and O^T += V^T P^T on
//     v_mfma_f32_16x16x32_f16 with the G heads on the N side (padded to 16);
//   - waves keep their own online-softmax state; the four are merged in LDS
//     and the splits by a small merge kernel.
// Probabilities enter the PV product as fp16 (q, K, V and P are not
// re-quantized; P rounding is within the tolerance of the plain definition).
#include "device_common.h"
#include "fp4_internal.h"

namespace fp4dev {

constexpr int kDecTile = 128;  // keys per staged tile
constexpr int kGmax = 16;      // query heads per kv head handled by one workgroup

// V^T rows (one per d) of a staged tile: row d starts at d * VS8 + dec_vpad(d / 16)
// 16-byte units.  The LDS has 32 four-byte banks; a wave's staging writes
// cover d rows 16 apart, which the one-unit row padding alone puts on the
// same banks.  The non-decreasing shift spreads them (rows never overlap);
// fragment reads take one 16-row group per instruction, so the shift is an
// immediate offset there.
template <int D>
__device__ __forceinline__ constexpr int dec_vpad(int grp) {
  return D == 128 ? 2 * grp : 4 * grp;
}

template <int D>
struct DecSmem {
  static constexpr int KS8 = D / 8 + 1;         // 16-byte units per K row (one unit of pad)
  static constexpr int VS8 = kDecTile / 8 + 1;  // 16-byte units per V^T row
  union {
    struct {
      half8_t k[kDecTile * KS8];
      half8_t v[D * VS8 + 16];
    };
    struct {  // wave-state merge, used after the last tile
      float red_m[4][kGmax];
      float red_l[4][kGmax];
      float red_o[4][kGmax][D];
    };
  };
};

// LDS of the FP4-region kernel: only V^T (K is consumed from registers).
template <int D>
struct DecSmemV {
  static constexpr int VS8 = kDecTile / 8 + 1;
  union {
    half8_t v[D * VS8 + 16];
    struct {
      float red_m[4][kGmax];
      float red_l[4][kGmax];
      float red_o[4][kGmax][D];
    };
  };
};

template <int D>
struct DecFetch {
  static constexpr int NCH = kDecTile * D / 32;
  static constexpr int PER = (NCH + 255) / 256;
  uint4_t kc[PER];
  uint32_t ks[PER];
  uint4_t vc[PER];
  uint4_t vs[PER];
};

__device__ __forceinline__ half2_t scale_h2(half2_t v, half_t s) { return v * half2_t{s, s}; }

template <int D>
__device__ __forceinline__ void dec_fetch(DecFetch<D>& F, const uint8_t* kc, const uint8_t* ks, const uint8_t* vc,
                                          const uint8_t* vs, int64_t key0, int64_t kend) {
#pragma unroll
  for (int u = 0; u < DecFetch<D>::PER; ++u) {
    const int q = threadIdx.x + 256 * u;
    if (q < DecFetch<D>::NCH) {
      const int kr = q / (D / 32), dc = q % (D / 32);
      const int64_t key = key0 + kr;
      if (key < kend) {
        F.kc[u] = *reinterpret_cast<const uint4_t*>(kc + key * (D / 2) + dc * 16);
        F.ks[u] = *reinterpret_cast<const uint16_t*>(ks + key * (D / 16) + dc * 2);
      } else {
        F.kc[u] = uint4_t{0, 0, 0, 0};
        F.ks[u] = 0;
      }
      const int pr = q / (D / 16), cc = q % (D / 16);
      const int64_t pair = key0 / 2 + pr;
      if (2 * pair < kend) {
        F.vc[u] = *reinterpret_cast<const uint4_t*>(vc + pair * D + cc * 16);
        F.vs[u] = *reinterpret_cast<const uint4_t*>(vs + (pair / 8) * D + cc * 16);
      } else {
        F.vc[u] = uint4_t{0, 0, 0, 0};
        F.vs[u] = uint4_t{0, 0, 0, 0};
      }
    }
  }
}

__device__ __forceinline__ half8_t dec_deq8(uint32_t cw, half_t s) {
  half2_t a = scale_h2(cvt_pk_f16_fp4<0>(cw), s), b = scale_h2(cvt_pk_f16_fp4<1>(cw), s);
  half2_t c = scale_h2(cvt_pk_f16_fp4<2>(cw), s), d = scale_h2(cvt_pk_f16_fp4<3>(cw), s);
  return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int D>
__device__ __forceinline__ void dec_stage_fp4(const DecFetch<D>& F, DecSmem<D>& S) {
  half2_t* v2 = reinterpret_cast<half2_t*>(S.v);
  constexpr int VS2 = DecSmem<D>::VS8 * 4;
#pragma unroll
  for (int u = 0; u < DecFetch<D>::PER; ++u) {
    const int q = threadIdx.x + 256 * u;
    if (q < DecFetch<D>::NCH) {
      const int kr = q / (D / 32), dc = q % (D / 32);
      const half2_t ks2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(F.ks[u], 1.0f, false);
      half8_t* dst = S.k + kr * DecSmem<D>::KS8 + dc * 4;
#pragma unroll
      for (int w = 0; w < 4; ++w) dst[w] = dec_deq8(F.kc[u][w], w < 2 ? ks2[0] : ks2[1]);
      const int pr = q / (D / 16), cc = q % (D / 16);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t cw = F.vc[u][w], sw = F.vs[u][w];
        const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
        const half2_t sb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true);
        const int col = 16 * cc + 4 * w;
        half2_t* dst = v2 + col * VS2 + 4 * dec_vpad<D>(cc) + pr;
        dst[0 * VS2] = scale_h2(cvt_pk_f16_fp4<0>(cw), sa[0]);
        dst[1 * VS2] = scale_h2(cvt_pk_f16_fp4<1>(cw), sa[1]);
        dst[2 * VS2] = scale_h2(cvt_pk_f16_fp4<2>(cw), sb[0]);
        dst[3 * VS2] = scale_h2(cvt_pk_f16_fp4<3>(cw), sb[1]);
      }
    }
  }
}

__device__ __forceinline__ half2_t bf16x2_to_half2(uint32_t w) {
  return half2_t{(half_t)__uint_as_float(w << 16), (half_t)__uint_as_float(w & 0xFFFF0000u)};
}

// bf16 tokens [k0, k0+128) of the full-precision part (sink then recent).
template <int D>
__device__ __forceinline__ void dec_stage_bf16(DecSmem<D>& S, const uint16_t* sink, const uint16_t* recent, int n_sink,
                                               int n_full, int64_t key0) {
  constexpr int NK = kDecTile * D / 8;
  for (int q = threadIdx.x; q < NK; q += 256) {
    const int kr = q / (D / 8), dc = q % (D / 8);
    const int64_t key = key0 + kr;
    uint4_t w = uint4_t{0, 0, 0, 0};
    if (key < n_full) {
      const uint16_t* src = key < n_sink ? sink + key * D : recent + (key - n_sink) * D;
      w = *reinterpret_cast<const uint4_t*>(src + dc * 8);
    }
    half2_t a = bf16x2_to_half2(w[0]), b = bf16x2_to_half2(w[1]), c = bf16x2_to_half2(w[2]), d2 = bf16x2_to_half2(w[3]);
    S.k[kr * DecSmem<D>::KS8 + dc] = half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d2[0], d2[1]};
  }
}
template <int D>
__device__ __forceinline__ void dec_stage_bf16_v(DecSmem<D>& S, const uint16_t* sink, const uint16_t* recent,
                                                 int n_sink, int n_full, int64_t key0) {
  constexpr int NV = (kDecTile / 2) * (D / 8);
  for (int q = threadIdx.x; q < NV; q += 256) {
    const int pr = q / (D / 8), cc = q % (D / 8);
    uint4_t w0 = uint4_t{0, 0, 0, 0}, w1 = uint4_t{0, 0, 0, 0};
    const int64_t key = key0 + 2 * pr;
    if (key < n_full) {
      const uint16_t* src = key < n_sink ? sink + key * D : recent + (key - n_sink) * D;
      w0 = *reinterpret_cast<const uint4_t*>(src + cc * 8);
    }
    if (key + 1 < n_full) {
      const uint16_t* src = key + 1 < n_sink ? sink + (key + 1) * D : recent + (key + 1 - n_sink) * D;
      w1 = *reinterpret_cast<const uint4_t*>(src + cc * 8);
    }
    half2_t* v2 = reinterpret_cast<half2_t*>(S.v);
    constexpr int VS2 = DecSmem<D>::VS8 * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half2_t a = bf16x2_to_half2(w0[j]), b = bf16x2_to_half2(w1[j]);
      const int col = cc * 8 + 2 * j;
      half2_t* dst = v2 + col * VS2 + 4 * dec_vpad<D>(col >> 4) + pr;
      dst[0] = half2_t{a[0], b[0]};
      dst[VS2] = half2_t{a[1], b[1]};
    }
  }
}

template <int D>
struct DecState {
  float4_t o[D / 16];  // O^T: d rows 16t + 4(lane/16) + i, head lane%16
  float m, l;          // per head (lane%16), l is this lane's part
};

// One wave's 32 keys of the staged tile: keys key0 + 32*wave .. +32 (valid < kend).
template <int D>
__device__ __forceinline__ void dec_wave_tile(const DecSmem<D>& S, const half8_t (&qf)[D / 32], DecState<D>& R,
                                              int64_t key0, int64_t kend, float c) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q4 = lane >> 4;  // lane group: holds keys 8*q4 .. 8*q4+7 of the wave's 32
  const int kw = 32 * wave;
  float4_t acc[2];
  acc[0] = float4_t{0, 0, 0, 0};
  acc[1] = float4_t{0, 0, 0, 0};
  // A row m of subtile g reads key 8*(m/4) + 4*g + m%4 (so lane group q4 ends up with keys 8*q4 .. +8)
  const int m = lane & 15;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int krow = kw + 8 * (m >> 2) + 4 * g + (m & 3);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const half8_t a = S.k[krow * DecSmem<D>::KS8 + 4 * s + q4];
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qf[s], acc[g], 0, 0, 0);
    }
  }
  // this lane: head lane%16, keys kw + 8*q4 + 4*g + i
  float x[8];
  float tm = -__builtin_inff();
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t key = key0 + kw + 8 * q4 + 4 * g + i;
      float v = acc[g][i] * c;
      if (key >= kend) v = -__builtin_inff();
      x[4 * g + i] = v;
      tm = __builtin_fmaxf(tm, v);
    }
  tm = __builtin_fmaxf(tm, __shfl_xor(tm, 16, 64));
  tm = __builtin_fmaxf(tm, __shfl_xor(tm, 32, 64));
  if (!(tm > -__builtin_inff())) return;  // whole 32-key slice beyond the context (uniform per head column)
  const float mnew = __builtin_fmaxf(R.m, tm);
  const float alpha = __builtin_amdgcn_exp2f(R.m - mnew);
  half8_t pf;
  float lsum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float e = __builtin_amdgcn_exp2f(x[j] - mnew);
    lsum += e;
    pf[j] = (half_t)e;
  }
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const half8_t a = S.v[(16 * t + (lane & 15)) * DecSmem<D>::VS8 + dec_vpad<D>(t) + kw / 8 + q4];
    R.o[t] = R.o[t] * alpha;
    R.o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pf, R.o[t], 0, 0, 0);
  }
  R.l = R.l * alpha + lsum;
  R.m = mnew;
}

struct DecArgs {
  const uint16_t* q;
  int64_t Hq, Hkv;
  int G, n_sink, n_recent;
  int64_t mid_cap, split_len;
  int nsplit;
  const uint16_t *k_sink, *v_sink, *k_recent, *v_recent;
  const uint8_t *kc, *ks, *vc, *vs;
  const int32_t* mid_len;
  float c;
  float* part_o;
  float* part_ml;
};

// ---- FP4 region: K straight from HBM into MFMA operands, V through LDS ----
//
// Each wave owns 32 keys of a 128-key tile.  For S^T = K q^T on
// v_mfma_f32_16x16x32_f16 the lanes of group q4 = lane/16 carry the d range
// [q4*D/4, (q4+1)*D/4) over the D/32 reduction steps (the B operand q uses the
// same d order), so one coalesced 16-byte load per lane (8 bytes for d = 64)
// brings a key's codes for all steps and K never touches LDS.  A-row m of
// subtile g reads key 8*(m/4) + 4*g + m%4, so each lane group ends up with 8
// consecutive keys, the order the PV step wants.  Only V goes through LDS
// (transposed to [d][key]), which halves LDS use and leaves room for more
// workgroups per CU; K and V codes are prefetched two tiles ahead.
template <int D>
struct KRegs {
  static constexpr int CB = D / 8;   // code bytes per lane per key (D/4 codes)
  static constexpr int SB = D / 64;  // scale bytes per lane per key
  uint32_t c[2][CB / 4];
  uint32_t s[2];
};

template <int D>
struct VRegs {
  static constexpr int NCH = kDecTile * D / 32;  // 16-byte chunks of V codes per tile
  static constexpr int PER = (NCH + 255) / 256;
  uint4_t c[PER];
  uint4_t s[PER];
};

// Loads go through buffer resources sized to the split's last token, so
// tokens past it read as zero (K: masked in the scores; V: zero rows) and no
// branch or clamp sits between loads -- several tiles stay in flight.
struct SplitBufs {
  rsrc_t kc, ks, vc, vs;
};

template <int D>
__device__ __forceinline__ void load_k(KRegs<D>& K, const SplitBufs& sb, int64_t key0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, m = lane & 15, q4 = lane >> 4;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const uint32_t key = (uint32_t)key0 + 32 * wave + 8 * (m >> 2) + 4 * g + (m & 3);
    if (D == 128) {
      const uint4_t w = buf_load16(sb.kc, key * (D / 2) + q4 * KRegs<D>::CB);
#pragma unroll
      for (int i = 0; i < KRegs<D>::CB / 4; ++i) K.c[g][i] = w[i];
      K.s[g] = buf_load2(sb.ks, key * (D / 16) + q4 * KRegs<D>::SB);
    } else {
      const uint2_t w = buf_load8(sb.kc, key * (D / 2) + q4 * KRegs<D>::CB);
#pragma unroll
      for (int i = 0; i < KRegs<D>::CB / 4; ++i) K.c[g][i] = w[i];
      K.s[g] = buf_load1(sb.ks, key * (D / 16) + q4 * KRegs<D>::SB);
    }
  }
}

template <int D>
__device__ __forceinline__ void load_v(VRegs<D>& V, const SplitBufs& sb, int64_t key0) {
#pragma unroll
  for (int u = 0; u < VRegs<D>::PER; ++u) {
    const int q = threadIdx.x + 256 * u;
    if (VRegs<D>::NCH % 256 == 0 || q < VRegs<D>::NCH) {
      const int pr = q / (D / 16), cc = q % (D / 16);
      const uint32_t pair = (uint32_t)(key0 / 2) + pr;
      V.c[u] = buf_load16(sb.vc, pair * D + cc * 16);
      V.s[u] = buf_load16(sb.vs, (pair / 8) * D + cc * 16);
    }
  }
}

template <int D>
__device__ __forceinline__ void stage_v(const VRegs<D>& V, DecSmemV<D>& S) {
  half2_t* v2 = reinterpret_cast<half2_t*>(S.v);
  constexpr int VS2 = DecSmemV<D>::VS8 * 4;
#pragma unroll
  for (int u = 0; u < VRegs<D>::PER; ++u) {
    const int q = threadIdx.x + 256 * u;
    if (q < VRegs<D>::NCH) {
      const int pr = q / (D / 16), cc = q % (D / 16);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t cw = V.c[u][w], sw = V.s[u][w];
        const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
        const half2_t sb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true);
        const int col = 16 * cc + 4 * w;
        half2_t* dst = v2 + col * VS2 + 4 * dec_vpad<D>(cc) + pr;
        dst[0 * VS2] = scale_h2(cvt_pk_f16_fp4<0>(cw), sa[0]);
        dst[1 * VS2] = scale_h2(cvt_pk_f16_fp4<1>(cw), sa[1]);
        dst[2 * VS2] = scale_h2(cvt_pk_f16_fp4<2>(cw), sb[0]);
        dst[3 * VS2] = scale_h2(cvt_pk_f16_fp4<3>(cw), sb[1]);
      }
    }
  }
}

// One wave's 32 keys: S^T from the K registers, softmax, O^T += V^T P^T.
template <int D>
__device__ __forceinline__ void fp4_wave_tile(const DecSmemV<D>& S, const KRegs<D>& K, const half8_t (&qf)[D / 32],
                                              DecState<D>& R, int64_t key0, int64_t kend, float c) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, q4 = lane >> 4;
  const int kw = 32 * wave;
  float4_t acc[2] = {float4_t{0, 0, 0, 0}, float4_t{0, 0, 0, 0}};
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const half2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(K.s[g], 1.0f, false);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const half_t sv = (s >> 1) == 0 ? sc[0] : sc[1];  // scale block of d = q4*D/4 + 8*s
      const half8_t a = dec_deq8(K.c[g][s], sv);
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qf[s], acc[g], 0, 0, 0);
    }
  }
  float x[8];
  float tm = -__builtin_inff();
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t key = key0 + kw + 8 * q4 + 4 * g + i;
      float v = acc[g][i] * c;
      if (key >= kend) v = -__builtin_inff();
      x[4 * g + i] = v;
      tm = __builtin_fmaxf(tm, v);
    }
  tm = __builtin_fmaxf(tm, __shfl_xor(tm, 16, 64));
  tm = __builtin_fmaxf(tm, __shfl_xor(tm, 32, 64));
  if (!(tm > -__builtin_inff())) return;
  const float mnew = __builtin_fmaxf(R.m, tm);
  const float alpha = __builtin_amdgcn_exp2f(R.m - mnew);
  half8_t pf;
  float lsum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float e = __builtin_amdgcn_exp2f(x[j] - mnew);
    lsum += e;
    pf[j] = (half_t)e;
  }
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const half8_t a = S.v[(16 * t + (lane & 15)) * DecSmemV<D>::VS8 + dec_vpad<D>(t) + kw / 8 + q4];
    R.o[t] = R.o[t] * alpha;
    R.o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pf, R.o[t], 0, 0, 0);
  }
  R.l = R.l * alpha + lsum;
  R.m = mnew;
}

// Merge the four waves' (m, l, O) in LDS and write this split's partial.
template <int D, typename SM>
__device__ __forceinline__ void write_partial(SM& S, const DecState<D>& R, const DecArgs& A, int64_t bk,
                                              int split) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, q4 = lane >> 4, head = lane & 15;
  const int ns1 = A.nsplit + 1;
  const float lh = R.l + __shfl_xor(R.l, 16, 64);
  const float lt = lh + __shfl_xor(lh, 32, 64);
  __syncthreads();
  if (q4 == 0) {
    S.red_m[wave][head] = R.m;
    S.red_l[wave][head] = lt;
  }
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) S.red_o[wave][head][16 * t + 4 * q4 + i] = R.o[t][i];
  __syncthreads();
  const int64_t pbase = bk * A.G;
  for (int idx = threadIdx.x; idx < A.G * D; idx += 256) {
    const int hh = idx / D, dd = idx % D;
    float mm = -__builtin_inff();
    for (int w = 0; w < 4; ++w) mm = __builtin_fmaxf(mm, S.red_m[w][hh]);
    float o = 0.0f, l = 0.0f;
    if (mm > -__builtin_inff())
      for (int w = 0; w < 4; ++w)
        if (S.red_m[w][hh] > -__builtin_inff()) {
          const float f = __builtin_amdgcn_exp2f(S.red_m[w][hh] - mm);
          o += S.red_o[w][hh][dd] * f;
          l += S.red_l[w][hh] * f;
        }
    A.part_o[((pbase + hh) * ns1 + split) * D + dd] = o;
    if (dd == 0) {
      A.part_ml[((pbase + hh) * ns1 + split) * 2] = mm;
      A.part_ml[((pbase + hh) * ns1 + split) * 2 + 1] = l;
    }
  }
}

template <int D>
__device__ __forceinline__ void load_q(half8_t (&qf)[D / 32], const DecArgs& A, int64_t bk) {
  const int lane = threadIdx.x & 63, q4 = lane >> 4, head = lane & 15;
  const bool ok = head < A.G;
  const uint16_t* qp = A.q + (bk * A.G + (ok ? head : 0)) * D + q4 * (D / 4);
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    uint4_t w = ok ? *reinterpret_cast<const uint4_t*>(qp + 8 * s) : uint4_t{0, 0, 0, 0};
    half2_t a = bf16x2_to_half2(w[0]), bb = bf16x2_to_half2(w[1]), cc = bf16x2_to_half2(w[2]), dd = bf16x2_to_half2(w[3]);
    qf[s] = half8_t{a[0], a[1], bb[0], bb[1], cc[0], cc[1], dd[0], dd[1]};
  }
}

// grid: (B*Hkv*nsplit); one workgroup per (batch, kv head, split of the FP4 region)
template <int D>
__global__ void __launch_bounds__(256, 3) decode_fp4_kernel(DecArgs A) {
  __shared__ DecSmemV<D> S;
  const int64_t gi = blockIdx.x;
  const int split = (int)(gi % A.nsplit);
  const int64_t bk = gi / A.nsplit;
  const int64_t b = bk / A.Hkv;
  half8_t qf[D / 32];
  load_q<D>(qf, A, bk);
  DecState<D> R;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) R.o[t] = float4_t{0, 0, 0, 0};
  R.m = -__builtin_inff();
  R.l = 0.0f;
  int64_t mlen = A.mid_len[b];
  if (mlen < 0) mlen = 0;
  if (mlen > A.mid_cap) mlen = A.mid_cap;
  mlen &= ~(int64_t)15;
  const int64_t s0 = (int64_t)split * A.split_len;
  int64_t s1 = s0 + A.split_len;
  if (s1 > mlen) s1 = mlen;
  // resources end at this split's last token s1 (a multiple of 16)
  SplitBufs sb;
  sb.kc = make_rsrc(A.kc + bk * A.mid_cap * (D / 2), (uint32_t)(s1 * (D / 2)));
  sb.ks = make_rsrc(A.ks + bk * A.mid_cap * (D / 16), (uint32_t)(s1 * (D / 16)));
  sb.vc = make_rsrc(A.vc + bk * (A.mid_cap / 2) * D, (uint32_t)((s1 / 2) * D));
  sb.vs = make_rsrc(A.vs + bk * (A.mid_cap / 16) * D, (uint32_t)((s1 / 16) * D));
  if (s0 < s1) {
    // tiles start at s0 + i*128; past the last one the prefetch reloads the
    // last tile (clamped, cached) instead of branching
    const int64_t last = s0 + ((s1 - s0 - 1) / kDecTile) * kDecTile;
    auto tclamp = [&](int64_t k) { return k < last ? k : last; };
    KRegs<D> K0, K1;
    VRegs<D> V0, V1;
    load_k<D>(K0, sb, s0);
    load_v<D>(V0, sb, s0);
    load_k<D>(K1, sb, tclamp(s0 + kDecTile));
    load_v<D>(V1, sb, tclamp(s0 + kDecTile));
    for (int64_t key0 = s0; key0 < s1; key0 += 2 * kDecTile) {
      // tile key0 from buffers 0, then refill them two tiles ahead
      __syncthreads();
      stage_v<D>(V0, S);
      load_v<D>(V0, sb, tclamp(key0 + 2 * kDecTile));
      __syncthreads();
      fp4_wave_tile<D>(S, K0, qf, R, key0, s1, A.c);
      load_k<D>(K0, sb, tclamp(key0 + 2 * kDecTile));
      // tile key0 + 128 from buffers 1
      if (key0 + kDecTile < s1) {
        __syncthreads();
        stage_v<D>(V1, S);
        load_v<D>(V1, sb, tclamp(key0 + 3 * kDecTile));
        __syncthreads();
        fp4_wave_tile<D>(S, K1, qf, R, key0 + kDecTile, s1, A.c);
        load_k<D>(K1, sb, tclamp(key0 + 3 * kDecTile));
      }
    }
  }
  write_partial<D>(S, R, A, bk, split);
}

// grid: (B*Hkv); the bf16 sink and recent tokens, written as split index nsplit.
template <int D>
__global__ void __launch_bounds__(256, 2) decode_full_kernel(DecArgs A) {
  __shared__ DecSmem<D> S;
  const int64_t bk = blockIdx.x;  // b * Hkv + kvh
  half8_t qf[D / 32];
  {
    // natural d order here (K comes through LDS)
    const int lane = threadIdx.x & 63, q4 = lane >> 4, head = lane & 15;
    const bool ok = head < A.G;
    const uint16_t* qp = A.q + (bk * A.G + (ok ? head : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      uint4_t w = ok ? *reinterpret_cast<const uint4_t*>(qp + 32 * s + 8 * q4) : uint4_t{0, 0, 0, 0};
      half2_t a = bf16x2_to_half2(w[0]), bb = bf16x2_to_half2(w[1]), cc = bf16x2_to_half2(w[2]), dd = bf16x2_to_half2(w[3]);
      qf[s] = half8_t{a[0], a[1], bb[0], bb[1], cc[0], cc[1], dd[0], dd[1]};
    }
  }
  DecState<D> R;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) R.o[t] = float4_t{0, 0, 0, 0};
  R.m = -__builtin_inff();
  R.l = 0.0f;
  const int n_full = A.n_sink + A.n_recent;
  const uint16_t* ksk = A.k_sink + bk * (int64_t)A.n_sink * D;
  const uint16_t* vsk = A.v_sink + bk * (int64_t)A.n_sink * D;
  const uint16_t* krc = A.k_recent + bk * (int64_t)A.n_recent * D;
  const uint16_t* vrc = A.v_recent + bk * (int64_t)A.n_recent * D;
  for (int64_t key0 = 0; key0 < n_full; key0 += kDecTile) {
    __syncthreads();
    dec_stage_bf16<D>(S, ksk, krc, A.n_sink, n_full, key0);
    dec_stage_bf16_v<D>(S, vsk, vrc, A.n_sink, n_full, key0);
    __syncthreads();
    dec_wave_tile<D>(S, qf, R, key0, n_full, A.c);
  }
  write_partial<D>(S, R, A, bk, A.nsplit);
}

template <typename OT>
__device__ __forceinline__ void store1(OT* p, float v);
template <>
__device__ __forceinline__ void store1<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store1<half_t>(half_t* p, float v) { *p = (half_t)v; }
template <>
__device__ __forceinline__ void store1<uint16_t>(uint16_t* p, float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7F800000u) != 0x7F800000u) u += 0x7FFFu + ((u >> 16) & 1u);
  *p = (uint16_t)(u >> 16);
}

// grid: B*Hq rows; block: D threads.
template <int D, typename OT>
__global__ void __launch_bounds__(128) decode_merge_kernel(const float* part_o, const float* part_ml, int ns1, OT* out,
                                                           float* lse) {
  const int64_t row = blockIdx.x;  // (b*Hkv + kvh) * G + g  ==  b*Hq + h
  const int dd = threadIdx.x;
  const float* ml = part_ml + row * ns1 * 2;
  float mm = -__builtin_inff();
  for (int s = 0; s < ns1; ++s) mm = __builtin_fmaxf(mm, ml[2 * s]);
  float o = 0.0f, l = 0.0f;
  if (mm > -__builtin_inff())
    for (int s = 0; s < ns1; ++s) {
      const float m = ml[2 * s];
      if (m > -__builtin_inff()) {
        const float w = __builtin_amdgcn_exp2f(m - mm);
        o += part_o[(row * ns1 + s) * D + dd] * w;
        l += ml[2 * s + 1] * w;
      }
    }
  store1<OT>(out + row * D + dd, l > 0.0f ? o / l : 0.0f);
  if (lse && dd == 0) lse[row] = l > 0.0f ? (mm + __builtin_log2f(l)) * 0.69314718055994531f : -__builtin_inff();
}

template <int D>
hipError_t launch_decode_d(const DecodeLaunch& L, hipStream_t st) {
  DecArgs A;
  A.q = (const uint16_t*)L.q;
  A.Hq = L.Hq;
  A.Hkv = L.Hkv;
  A.G = (int)(L.Hq / L.Hkv);
  A.n_sink = L.n_sink;
  A.n_recent = L.n_recent;
  A.mid_cap = L.mid_cap;
  A.split_len = L.split_len;
  A.nsplit = L.nsplit;
  A.k_sink = (const uint16_t*)L.k_sink;
  A.v_sink = (const uint16_t*)L.v_sink;
  A.k_recent = (const uint16_t*)L.k_recent;
  A.v_recent = (const uint16_t*)L.v_recent;
  A.kc = L.kc; A.ks = L.ks; A.vc = L.vc; A.vs = L.vs;
  A.mid_len = L.mid_len;
  A.c = L.c;
  A.part_o = L.part_o;
  A.part_ml = L.part_ml;
  const int ns1 = L.nsplit + 1;
  if (L.nsplit > 0)
    hipLaunchKernelGGL(decode_fp4_kernel<D>, dim3((unsigned)(L.B * L.Hkv * L.nsplit)), dim3(256), 0, st, A);
  hipLaunchKernelGGL(decode_full_kernel<D>, dim3((unsigned)(L.B * L.Hkv)), dim3(256), 0, st, A);
  const dim3 mg((unsigned)(L.B * L.Hq));
  if (L.out_dtype == 2)
    hipLaunchKernelGGL((decode_merge_kernel<D, float>), mg, dim3(D), 0, st, L.part_o, L.part_ml, ns1, (float*)L.out, L.lse);
  else if (L.out_dtype == 1)
    hipLaunchKernelGGL((decode_merge_kernel<D, half_t>), mg, dim3(D), 0, st, L.part_o, L.part_ml, ns1, (half_t*)L.out, L.lse);
  else
    hipLaunchKernelGGL((decode_merge_kernel<D, uint16_t>), mg, dim3(D), 0, st, L.part_o, L.part_ml, ns1, (uint16_t*)L.out, L.lse);
  return hipGetLastError();
}

}  // namespace fp4dev

using namespace fp4dev;

int fp4i_decode_splits(int64_t B, int64_t Hkv, int64_t mid_cap, int64_t* split_len) {
  if (mid_cap <= 0) {
    *split_len = kDecTile;
    return 0;
  }
  const int64_t tiles = (mid_cap + kDecTile - 1) / kDecTile;
  int64_t want = (2048 + B * Hkv - 1) / (B * Hkv);  // splits per (b, kvh) to reach ~2048 workgroups
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  const int64_t tiles_per = (tiles + want - 1) / want;
  *split_len = tiles_per * kDecTile;
  return (int)((mid_cap + *split_len - 1) / *split_len);
}

hipError_t fp4i_launch_decode(const DecodeLaunch& L, hipStream_t st) {
  if (L.d == 128) return launch_decode_d<128>(L, st);
  return launch_decode_d<64>(L, st);
}

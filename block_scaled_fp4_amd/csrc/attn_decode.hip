// attn_decode.hip -- one-token decode over a sink-aware mixed-precision KV
// cache (ScaleSearch page, Metodologia / ScaleSearchAttention: the first and
// last cache blocks stay in full precision, the rest in NVFP4).
//
// Decode is bound by HBM: every cached byte is read once per step and used by
// only the G = Hq/Hkv query heads of its group.  MI355X mapping:
//   - the FP4 region of every (batch, kv head) is split over workgroups of
//     four waves; each wave streams its own contiguous run of keys, 32 keys a
//     step, with no LDS and no barrier until the final merge, keeping two
//     steps of loads in flight;
//   - S^T = K q^T and O^T += V^T P^T run on v_mfma_f32_16x16x32_f16 with the G
//     heads on the N side (padded to 16); every operand is dequantized in
//     registers (code * E4M3 scale is exact in fp16);
//   - K: lane group q4 = lane/16 covers d range [q4*D/4, (q4+1)*D/4) of the
//     reduction order shared with q, so one coalesced 16-byte load per lane
//     and key feeds all steps;
//   - V is stored with two tokens per code byte (blocks of 16 tokens).  A lane
//     loads D/16 consecutive channels of four token pairs and a 4x4 byte
//     transpose (v_perm_b32) turns them into one dword of 8 consecutive
//     tokens per channel -- exactly an A-operand row of the PV product;
//   - extra workgroups of the same launch read the bf16 sink and recent
//     tokens (128 per workgroup); the waves of a workgroup merge their
//     (m, l, O) in LDS and a second kernel merges the workgroups' partials;
//   - with selective promotion (ThriftAttention page, Metodologia / 2, in
//     decode) a selection kernel first picks middle blocks of 128 tokens;
//     further workgroups read those blocks from the full-precision copy (one
//     block per wave), and the FP4 waves skip them: their loads fall past the
//     buffer resources' ends (no memory access) and their keys are masked.
// Probabilities enter the PV product as fp16 (q, K, V and P are not
// re-quantized; P rounding is within the tolerance of the plain definition).
#include "device_common.h"
#include "fp4_internal.h"

namespace fp4dev {

constexpr int kStep = 32;     // keys per wave step
constexpr int kDecWaves = 4;  // waves per workgroup
constexpr int kGmax = 16;     // query heads per kv head handled by one workgroup

// The reference exponent of a head moves only when a step's maximum exceeds
// it by more than kDecRaise, so p = 2^(x - m) <= 2^kDecRaise stays in fp16.
constexpr float kDecRaise = 8.0f;

// Per-wave state.  O^T of PV MFMA t: this lane holds channels
// d = (D/16) * (4*(lane/16) + r) + t, r = 0..3, of head lane%16.
template <int D>
struct DecState {
  float4_t o[D / 16];
  float m;  // reference exponent (x units) of head lane%16
  float l;  // this lane's part of the denominator, relative to 2^m
};

// Cross-wave merge buffers of one workgroup.
template <int D>
struct DecRed {
  float m[kDecWaves][kGmax];
  float l[kDecWaves][kGmax];
  float o[kDecWaves][kGmax][D];
};

// One step's quantized K and V in registers.
template <int D>
struct KStep {
  uint32_t c[2][D / 32];  // subtile g: the lane's D/4 codes of one key
  uint32_t s[2];          // its D/64 scale bytes
};
template <int D>
struct VStep {
  uint32_t c[4][D / 64];  // token pair r: D/16 channel bytes (two tokens each)
  uint32_t s[D / 64];     // the D/16 channels' scale bytes of the lane's 16-token block
};

struct DecArgs {
  const uint16_t* q;
  int64_t Hq, Hkv, nbk;  // nbk = B * Hkv
  int G, n_sink, n_recent;
  int64_t mid_cap, split_len;
  int nsplit, nfull, ns1;  // FP4 splits, full-precision workgroups, partials per row (their sum)
  const uint16_t *k_sink, *v_sink, *k_recent, *v_recent;
  const uint8_t *kc, *ks, *vc, *vs;
  const int32_t* mid_len;
  float c;
  float* part_o;
  float* part_ml;
  // selective promotion: workgroups of four promoted blocks (one per wave)
  const uint16_t *k_mid, *v_mid;  // full-precision copy of the middle
  const int32_t* sel_idx;         // [nbk, kmax] promoted blocks, -1 padded
  const uint32_t* sel_mask;       // [nbk, nbw] bit j: block j promoted (null: none)
  int kmax, nprom, nbw;
};

struct SplitBufs {
  rsrc_t kc, ks, vc, vs;
};

__device__ __forceinline__ half2_t scale_h2(half2_t v, half_t s) { return v * half2_t{s, s}; }

// 8 E2M1 codes (one dword, low nibble first) times one fp16 scale.
__device__ __forceinline__ half8_t dec_deq8(uint32_t cw, half_t s) {
  half2_t a = scale_h2(cvt_pk_f16_fp4<0>(cw), s), b = scale_h2(cvt_pk_f16_fp4<1>(cw), s);
  half2_t c = scale_h2(cvt_pk_f16_fp4<2>(cw), s), d = scale_h2(cvt_pk_f16_fp4<3>(cw), s);
  return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ half2_t bf16x2_to_half2(uint32_t w) {
  return half2_t{(half_t)__uint_as_float(w << 16), (half_t)__uint_as_float(w & 0xFFFF0000u)};
}

// 4x4 byte transpose: o[j] = byte j of a, b, c, d (in that order).  v_perm_b32
// selects bytes of {S0:S1}, S1 being bytes 0-3.
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

// K subtile row m of subtile g holds key 8*(m/4) + 4*g + m%4 of the step, so
// the S^T output leaves lane group q4 with the 8 consecutive keys 8*q4 .. +8,
// the order the P^T operand of the PV product wants.
__device__ __forceinline__ uint32_t krow(int m, int g) { return 8u * (m >> 2) + 4u * g + (m & 3); }

// Loads go through buffer resources that end at the split's last token, so
// nothing past it is read (zeros come back) and no branch sits between loads.
template <int D>
__device__ __forceinline__ void load_fp4(KStep<D>& K, VStep<D>& V, const SplitBufs& sb, uint32_t key0) {
  const int lane = threadIdx.x & 63, m = lane & 15, q4 = lane >> 4;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const uint32_t key = key0 + krow(m, g);
    if (D == 128) {
      const uint4_t w = buf_load16(sb.kc, key * 64u + q4 * 16u);
#pragma unroll
      for (int i = 0; i < 4; ++i) K.c[g][i] = w[i];
      K.s[g] = buf_load2(sb.ks, key * 8u + q4 * 2u);
    } else {
      const uint2_t w = buf_load8(sb.kc, key * 32u + q4 * 8u);
      K.c[g][0] = w[0];
      K.c[g][1] = w[1];
      K.s[g] = buf_load1(sb.ks, key * 4u + q4);
    }
  }
  // V: lane (channel group m, key group q4): token pairs key0/2 + 4*q4 + r
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t pair = key0 / 2u + 4u * q4 + r;
    if (D == 128) {
      const uint2_t w = buf_load8(sb.vc, pair * 128u + 8u * m);
      V.c[r][0] = w[0];
      V.c[r][1] = w[1];
    } else {
      V.c[r][0] = buf_load4(sb.vc, pair * 64u + 4u * m);
    }
  }
  const uint32_t blk = key0 / 16u + (q4 >> 1);
  if (D == 128) {
    const uint2_t w = buf_load8(sb.vs, blk * 128u + 8u * m);
    V.s[0] = w[0];
    V.s[1] = w[1];
  } else {
    V.s[0] = buf_load4(sb.vs, blk * 64u + 4u * m);
  }
}

// Softmax of one step: x = S c (keys >= kend masked), lazy reference update,
// p = 2^(x - m) as the fp16 P^T operand (returned); updates R.
template <int D>
__device__ __forceinline__ half8_t step_softmax(const float4_t (&acc)[2], uint32_t key0, uint32_t kend, float c,
                                                DecState<D>& R) {
  const int lane = threadIdx.x & 63, q4 = lane >> 4;
  float x[8];
  float tm = -__builtin_inff();
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t key = key0 + 8u * q4 + 4u * g + i;
      float v = acc[g][i] * c;
      if (key >= kend) v = -__builtin_inff();
      x[4 * g + i] = v;
      tm = __builtin_fmaxf(tm, v);
    }
  tm = __builtin_fmaxf(tm, __shfl_xor(tm, 16, 64));
  tm = __builtin_fmaxf(tm, __shfl_xor(tm, 32, 64));
  const bool raise = tm > R.m + kDecRaise;  // R.m = -inf: any finite maximum raises
  if (__any(raise)) {
    const float f = raise ? __builtin_amdgcn_exp2f(R.m - tm) : 1.0f;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) R.o[t] = R.o[t] * f;
    R.l = R.l * f;
    if (raise) R.m = tm;
  }
  const float off = R.m > -__builtin_inff() ? R.m : 0.0f;
  half8_t pf;
  float lsum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = __builtin_amdgcn_exp2f(x[j] - off);
    lsum += p;
    pf[j] = (half_t)p;
  }
  R.l += lsum;
  return pf;
}

template <int D>
__device__ __forceinline__ void fp4_step(const KStep<D>& K, const VStep<D>& V, const half8_t (&qf)[D / 32],
                                         DecState<D>& R, uint32_t key0, uint32_t kend, float c) {
  float4_t acc[2] = {float4_t{0, 0, 0, 0}, float4_t{0, 0, 0, 0}};
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const half2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(K.s[g], 1.0f, false);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const half_t sv = (s >> 1) == 0 ? sc[0] : sc[1];  // scale block of d = q4*D/4 + 8*s
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dec_deq8(K.c[g][s], sv), qf[s], acc[g], 0, 0, 0);
    }
  }
  // V^T operands: channel (D/16)*m + t, keys 8*q4 .. +8
  uint32_t tc[D / 16];
#pragma unroll
  for (int u = 0; u < D / 64; ++u) transpose4(V.c[0][u], V.c[1][u], V.c[2][u], V.c[3][u], tc + 4 * u);
  half_t sv[D / 16];
#pragma unroll
  for (int u = 0; u < D / 64; ++u) {
    const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(V.s[u], 1.0f, false);
    const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(V.s[u], 1.0f, true);
    sv[4 * u] = a[0];
    sv[4 * u + 1] = a[1];
    sv[4 * u + 2] = b[0];
    sv[4 * u + 3] = b[1];
  }
  const half8_t pf = step_softmax<D>(acc, key0, kend, c, R);
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    R.o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dec_deq8(tc[t], sv[t]), pf, R.o[t], 0, 0, 0);
}

// One step of the full-precision (bf16) tokens: key k < n_sink is sink[k],
// else recent[k - n_sink]; keys >= n_full are masked.
template <int D>
__device__ __forceinline__ const uint16_t* full_row(const uint16_t* sink, const uint16_t* recent, int n_sink,
                                                    uint32_t key) {
  return (int)key < n_sink ? sink + (size_t)key * D : recent + (size_t)(key - n_sink) * D;
}

template <int D>
__device__ __forceinline__ void bf16_step(const uint16_t* ksk, const uint16_t* krc, const uint16_t* vsk,
                                          const uint16_t* vrc, int n_sink, uint32_t n_full,
                                          const half8_t (&qf)[D / 32], DecState<D>& R, uint32_t key0, float c) {
  const int lane = threadIdx.x & 63, m = lane & 15, q4 = lane >> 4;
  float4_t acc[2] = {float4_t{0, 0, 0, 0}, float4_t{0, 0, 0, 0}};
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const uint32_t key = key0 + krow(m, g);
    const bool ok = key < n_full;
    const uint16_t* src = full_row<D>(ksk, krc, n_sink, ok ? key : 0u) + 8 * q4;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      // reduction order of the bf16 tokens: lane group q4, step s -> d = 8 (q4 + 4 s) .. +8,
      // so the four lane groups read 64 contiguous bytes of a key row per load
      const uint4_t w = ok ? *reinterpret_cast<const uint4_t*>(src + 32 * s) : uint4_t{0, 0, 0, 0};
      const half2_t a = bf16x2_to_half2(w[0]), b = bf16x2_to_half2(w[1]);
      const half2_t cc = bf16x2_to_half2(w[2]), dd = bf16x2_to_half2(w[3]);
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(half8_t{a[0], a[1], b[0], b[1], cc[0], cc[1], dd[0], dd[1]},
                                                      qf[s], acc[g], 0, 0, 0);
    }
  }
  // V^T operand t: channel (D/16)*m + t, keys 8*q4 + j
  half8_t vf[D / 16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t key = key0 + 8u * q4 + j;
    const bool ok = key < n_full;
    const uint16_t* src = full_row<D>(vsk, vrc, n_sink, ok ? key : 0u) + (D / 16) * m;
    uint32_t w[D / 32];
    if (D == 128) {
      const uint4_t x = ok ? *reinterpret_cast<const uint4_t*>(src) : uint4_t{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < D / 32; ++i) w[i] = x[i];
    } else {
      const uint2_t x = ok ? *reinterpret_cast<const uint2_t*>(src) : uint2_t{0, 0};
#pragma unroll
      for (int i = 0; i < D / 32; ++i) w[i] = x[i];
    }
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const half2_t h = bf16x2_to_half2(w[i]);
      vf[2 * i][j] = h[0];
      vf[2 * i + 1][j] = h[1];
    }
  }
  const half8_t pf = step_softmax<D>(acc, key0, n_full, c, R);
#pragma unroll
  for (int t = 0; t < D / 16; ++t) R.o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[t], pf, R.o[t], 0, 0, 0);
}

// q fragments in the K reduction order: lane group q4, step s -> d = q4*D/4 + 8*s .. +8
// for the NVFP4 keys (FULL false), d = 8 (q4 + 4 s) .. +8 for the bf16 ones.
template <int D, bool FULL = false>
__device__ __forceinline__ void load_q(half8_t (&qf)[D / 32], const DecArgs& A, int64_t bk) {
  const int lane = threadIdx.x & 63, q4 = lane >> 4, head = lane & 15;
  const bool ok = head < A.G;
  const uint16_t* qp = A.q + (bk * A.G + (ok ? head : 0)) * D + (FULL ? 8 * q4 : q4 * (D / 4));
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    uint4_t w = ok ? *reinterpret_cast<const uint4_t*>(qp + (FULL ? 32 : 8) * s) : uint4_t{0, 0, 0, 0};
    half2_t a = bf16x2_to_half2(w[0]), bb = bf16x2_to_half2(w[1]), cc = bf16x2_to_half2(w[2]), dd = bf16x2_to_half2(w[3]);
    qf[s] = half8_t{a[0], a[1], bb[0], bb[1], cc[0], cc[1], dd[0], dd[1]};
  }
}

// Merge the waves' (m, l, O) in LDS and write this split's partial.
template <int D>
__device__ __forceinline__ void write_partial(DecRed<D>& S, const DecState<D>& R, const DecArgs& A, int64_t bk,
                                              int split) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, q4 = lane >> 4, head = lane & 15;
  const int ns1 = A.ns1;
  const float lh = R.l + __shfl_xor(R.l, 16, 64);
  const float lt = lh + __shfl_xor(lh, 32, 64);
  if (q4 == 0) {
    S.m[wave][head] = R.m;
    S.l[wave][head] = lt;
  }
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) S.o[wave][head][(D / 16) * (4 * q4 + r) + t] = R.o[t][r];
  __syncthreads();
  const int64_t pbase = bk * A.G;
  for (int idx = threadIdx.x; idx < A.G * D; idx += 64 * kDecWaves) {
    const int hh = idx / D, dd = idx % D;
    float mm = -__builtin_inff();
    for (int w = 0; w < kDecWaves; ++w) mm = __builtin_fmaxf(mm, S.m[w][hh]);
    float o = 0.0f, l = 0.0f;
    if (mm > -__builtin_inff())
      for (int w = 0; w < kDecWaves; ++w)
        if (S.m[w][hh] > -__builtin_inff()) {
          const float f = __builtin_amdgcn_exp2f(S.m[w][hh] - mm);
          o += S.o[w][hh][dd] * f;
          l += S.l[w][hh] * f;
        }
    A.part_o[((pbase + hh) * ns1 + split) * D + dd] = o;
    if (dd == 0) {
      A.part_ml[((pbase + hh) * ns1 + split) * 2] = mm;
      A.part_ml[((pbase + hh) * ns1 + split) * 2 + 1] = l;
    }
  }
}

// Workgroup f of a (batch, kv head) over its full-precision tokens
// [128 f, 128 f + 128), one step per wave; partial index nsplit + f.
template <int D>
__device__ __forceinline__ void full_workgroup(DecRed<D>& S, const DecArgs& A, int64_t bk, int f, int wave) {
  half8_t qf[D / 32];
  load_q<D, true>(qf, A, bk);
  DecState<D> R;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) R.o[t] = float4_t{0, 0, 0, 0};
  R.m = -__builtin_inff();
  R.l = 0.0f;
  const uint32_t n_full = (uint32_t)(A.n_sink + A.n_recent);
  const uint32_t key0 = (uint32_t)(kStep * kDecWaves * f + kStep * wave);
  if (key0 < n_full) {
    const uint16_t* ksk = A.k_sink + bk * (int64_t)A.n_sink * D;
    const uint16_t* vsk = A.v_sink + bk * (int64_t)A.n_sink * D;
    const uint16_t* krc = A.k_recent + bk * (int64_t)A.n_recent * D;
    const uint16_t* vrc = A.v_recent + bk * (int64_t)A.n_recent * D;
    bf16_step<D>(ksk, krc, vsk, vrc, A.n_sink, n_full, qf, R, key0, A.c);
  }
  write_partial<D>(S, R, A, bk, A.nsplit + f);
}

// Workgroup f of the promoted blocks of a (batch, kv head): wave w reads
// promoted block sel_idx[4 f + w] (128 tokens, fewer for a short last block)
// from the full-precision copy; partial index nsplit + nfull + f.
template <int D>
__device__ __forceinline__ void promoted_workgroup(DecRed<D>& S, const DecArgs& A, int64_t bk, int f, int wave) {
  half8_t qf[D / 32];
  load_q<D, true>(qf, A, bk);
  DecState<D> R;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) R.o[t] = float4_t{0, 0, 0, 0};
  R.m = -__builtin_inff();
  R.l = 0.0f;
  const int slot = 4 * f + wave;
  const int j = slot < A.kmax ? A.sel_idx[bk * A.kmax + slot] : -1;
  if (j >= 0) {
    int64_t mlen = A.mid_len[bk / A.Hkv];
    if (mlen < 0) mlen = 0;
    if (mlen > A.mid_cap) mlen = A.mid_cap;
    mlen &= ~(int64_t)15;
    const int64_t t0 = (int64_t)j * (kStep * kDecWaves);
    const int64_t rest = mlen - t0;
    const uint32_t n = (uint32_t)(rest < kStep * kDecWaves ? (rest > 0 ? rest : 0) : kStep * kDecWaves);
    const uint16_t* kb = A.k_mid + (bk * A.mid_cap + t0) * D;
    const uint16_t* vb = A.v_mid + (bk * A.mid_cap + t0) * D;
    for (uint32_t key0 = 0; key0 < n; key0 += kStep) bf16_step<D>(kb, kb, vb, vb, 0, n, qf, R, key0, A.c);
  }
  write_partial<D>(S, R, A, bk, A.nsplit + A.nfull + f);
}

// grid: B*Hkv*nfull workgroups over the full-precision (bf16 sink + recent)
// tokens, B*Hkv*nprom over the promoted middle blocks, then B*Hkv*nsplit over
// the splits of the FP4 region of each (batch, kv head) (partial index =
// split).  (The short promoted workgroups go before the long splits: the
// other order measured 10% slower.)
template <int D>
__global__ void __launch_bounds__(64 * kDecWaves, 3) decode_kernel(DecArgs A) {
  __shared__ DecRed<D> S;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t nfw = A.nbk * A.nfull;
  if ((int64_t)blockIdx.x < nfw) {
    // (its own scope, returning: the two kinds of workgroup share no
    // registers, so the rare bf16 one does not raise the kernel's count)
    full_workgroup<D>(S, A, (int64_t)blockIdx.x / A.nfull, (int)((int64_t)blockIdx.x % A.nfull), wave);
    return;
  }
  const int64_t npw = A.nbk * A.nprom;
  if ((int64_t)blockIdx.x - nfw < npw) {
    const int64_t gp = (int64_t)blockIdx.x - nfw;
    promoted_workgroup<D>(S, A, gp / A.nprom, (int)(gp % A.nprom), wave);
    return;
  }
  const int64_t gi = (int64_t)blockIdx.x - nfw - npw;
  const int64_t bk = gi / A.nsplit;
  const int split = (int)(gi % A.nsplit);
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
  // this wave's keys [ws, we): a quarter of the split (multiple of 32)
  const int64_t wl = A.split_len / kDecWaves;
  const int64_t ws = s0 + wave * wl;
  const int64_t we = ws + wl < s1 ? ws + wl : s1;
  if (ws < we) {
    // resources end at the split's last token s1 (a multiple of 16)
    SplitBufs sb;
    sb.kc = make_rsrc(A.kc + bk * A.mid_cap * (D / 2), (uint32_t)(s1 * (D / 2)));
    sb.ks = make_rsrc(A.ks + bk * A.mid_cap * (D / 16), (uint32_t)(s1 * (D / 16)));
    sb.vc = make_rsrc(A.vc + bk * (A.mid_cap / 2) * D, (uint32_t)((s1 / 2) * D));
    sb.vs = make_rsrc(A.vs + bk * (A.mid_cap / 16) * D, (uint32_t)((s1 / 16) * D));
    // steps of promoted blocks load from key kOOB instead: every offset then
    // lies at or past 2^28 (scales) or 2^31 (codes), beyond the resources'
    // ends (mid_cap * D / 2 < 2^31), so nothing is read and zeros come back;
    // their keys are masked
    constexpr uint32_t kOOB = (1u << 31) / (D / 2);
    const uint32_t* smask = A.sel_mask ? A.sel_mask + bk * A.nbw : nullptr;
    auto promoted = [&](uint32_t key) {
      if (!smask) return false;
      const uint32_t blk = key / (kStep * kDecWaves);
      const uint32_t word = (uint32_t)__builtin_amdgcn_readfirstlane((int)smask[blk >> 5]);  // wave-uniform
      return ((word >> (blk & 31u)) & 1u) != 0u;
    };
    auto at = [&](uint32_t key) { return promoted(key) ? kOOB : key; };
    auto stop = [&](uint32_t key) { return promoted(key) ? key : (uint32_t)we; };
    const uint32_t kend = (uint32_t)we;
    // steps start at ws + 32 i; prefetches past the last one reload it
    // (cached) instead of branching
    const uint32_t last = (uint32_t)(ws + ((we - ws - 1) / kStep) * kStep);
    auto clampk = [&](uint32_t k) { return k < last ? k : last; };
    KStep<D> K0, K1, K2;
    VStep<D> V0, V1, V2;
    load_fp4<D>(K0, V0, sb, at((uint32_t)ws));
    load_fp4<D>(K1, V1, sb, at(clampk((uint32_t)ws + kStep)));
    for (uint32_t key0 = (uint32_t)ws; key0 < kend; key0 += 3 * kStep) {
      load_fp4<D>(K2, V2, sb, at(clampk(key0 + 2 * kStep)));
      fp4_step<D>(K0, V0, qf, R, key0, stop(key0), A.c);
      if (key0 + kStep >= kend) break;
      load_fp4<D>(K0, V0, sb, at(clampk(key0 + 3 * kStep)));
      fp4_step<D>(K1, V1, qf, R, key0 + kStep, stop(key0 + kStep), A.c);
      if (key0 + 2 * kStep >= kend) break;
      load_fp4<D>(K1, V1, sb, at(clampk(key0 + 4 * kStep)));
      fp4_step<D>(K2, V2, qf, R, key0 + 2 * kStep, stop(key0 + 2 * kStep), A.c);
    }
  }
  write_partial<D>(S, R, A, bk, split);
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
  // (unrolled, loads unconditional, so that several partials are in flight at
  // once; an empty partial has m = -inf, l = 0, o = 0 and weight 0)
  float mm = -__builtin_inff();
#pragma unroll 8
  for (int s = 0; s < ns1; ++s) mm = __builtin_fmaxf(mm, ml[2 * s]);
  float o = 0.0f, l = 0.0f;
  if (mm > -__builtin_inff()) {
#pragma unroll 8
    for (int s = 0; s < ns1; ++s) {
      const float w = __builtin_amdgcn_exp2f(ml[2 * s] - mm);
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
  A.nbk = L.B * L.Hkv;
  A.G = (int)(L.Hq / L.Hkv);
  A.n_sink = L.n_sink;
  A.n_recent = L.n_recent;
  A.mid_cap = L.mid_cap;
  A.split_len = L.split_len;
  A.nsplit = L.nsplit;
  A.nfull = L.nfull;
  A.k_sink = (const uint16_t*)L.k_sink;
  A.v_sink = (const uint16_t*)L.v_sink;
  A.k_recent = (const uint16_t*)L.k_recent;
  A.v_recent = (const uint16_t*)L.v_recent;
  A.kc = L.kc; A.ks = L.ks; A.vc = L.vc; A.vs = L.vs;
  A.mid_len = L.mid_len;
  A.c = L.c;
  A.part_o = L.part_o;
  A.part_ml = L.part_ml;
  A.k_mid = (const uint16_t*)L.k_mid;
  A.v_mid = (const uint16_t*)L.v_mid;
  A.sel_idx = L.sel_idx;
  A.sel_mask = L.sel_mask;
  A.kmax = L.kmax;
  A.nprom = L.nprom;
  A.nbw = L.nbw;
  A.ns1 = L.nsplit + L.nfull + L.nprom;
  const int ns1 = A.ns1;
  hipLaunchKernelGGL(decode_kernel<D>, dim3((unsigned)(L.B * L.Hkv * ns1)), dim3(64 * kDecWaves), 0, st, A);
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

// Splits of the FP4 region per (batch, kv head): enough workgroups of four
// streaming waves (about 1024) to keep every CU's loads in flight.  A split
// is a multiple of 128 tokens, so each wave's quarter is a multiple of 32.
int fp4i_decode_splits(int64_t B, int64_t Hkv, int64_t mid_cap, int64_t* split_len) {
  constexpr int64_t kUnit = kStep * kDecWaves;
  if (mid_cap <= 0) {
    *split_len = kUnit;
    return 0;
  }
  const int64_t units = (mid_cap + kUnit - 1) / kUnit;
  int64_t want = (1024 + B * Hkv - 1) / (B * Hkv);
  if (want < 1) want = 1;
  if (want > units) want = units;
  const int64_t units_per = (units + want - 1) / want;
  *split_len = units_per * kUnit;
  return (int)((mid_cap + *split_len - 1) / *split_len);
}

// Workgroups of 128 full-precision tokens per (batch, kv head).
int fp4i_decode_full_splits(int64_t n_full) { return (int)((n_full + kStep * kDecWaves - 1) / (kStep * kDecWaves)); }

hipError_t fp4i_launch_decode(const DecodeLaunch& L, hipStream_t st) {
  if (L.d == 128) return launch_decode_d<128>(L, st);
  return launch_decode_d<64>(L, st);
}

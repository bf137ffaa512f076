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
// One pass recomputes the scores and writes P^ and dS (one float per
// query/key pair each, so the workspace grows with B H Sq Sk); dV, dQ and dK
// are batched GEMMs on the bf16 MFMA with binary32 accuracy (128 x 128 tiles,
// LDS staged), the query heads of a kv head being consecutive rows of one
// GEMM for dK and dV.
#include "device_common.h"
#include "fp4_internal.h"

namespace fp4dev {

constexpr int kGT = 128;  // output tile (M and N) of the products

// ---- operands in fp32 ----------------------------------------------------

// NVFP4 rows with blocks along the row (Q, K): codes [rows, d/2], scales
// [rows, d/16] -> fp32 [rows, d].  One thread per 8 codes (4 bytes).
__global__ void __launch_bounds__(256) dequant_rows_kernel(const uint8_t* codes, const uint8_t* scales,
                                                           int64_t rows, int d, float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // group of 8 elements
  const int64_t n = rows * (d / 8);
  if (i >= n) return;
  const int64_t r = i / (d / 8);
  const int c8 = (int)(i % (d / 8));
  const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + r * (d / 2) + 4 * c8);
  const float s = e4m3_to_f32(scales[r * (d / 16) + c8 / 2]);
  float* o = out + r * d + 8 * c8;
  const float2_t v0 = cvt_pk_f32_fp4<0>(w), v1 = cvt_pk_f32_fp4<1>(w);
  const float2_t v2 = cvt_pk_f32_fp4<2>(w), v3 = cvt_pk_f32_fp4<3>(w);
  *reinterpret_cast<float4_t*>(o) = float4_t{v0[0] * s, v0[1] * s, v1[0] * s, v1[1] * s};
  *reinterpret_cast<float4_t*>(o + 4) = float4_t{v2[0] * s, v2[1] * s, v3[0] * s, v3[1] * s};
}

// NVFP4 with blocks of 16 rows (V): codes [rows/2, d] (row 2i in the low
// nibble), scales [rows/16, d] -> fp32 [rows, d].  One thread per row pair
// and column.
__global__ void __launch_bounds__(256) dequant_cols_kernel(const uint8_t* codes, const uint8_t* scales,
                                                           int64_t rows, int d, float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (rows / 2) * d;
  if (i >= n) return;
  const int64_t pr = i / d;
  const int c = (int)(i % d);
  const uint32_t b = codes[pr * d + c];
  const float s = e4m3_to_f32(scales[(pr / 8) * d + c]);
  const float2_t v = cvt_pk_f32_fp4<0>(b);
  out[(2 * pr) * d + c] = v[0] * s;
  out[(2 * pr + 1) * d + c] = v[1] * s;
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }
template <>
__device__ __forceinline__ float to_f32<half_t>(half_t v) { return (float)v; }
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }

template <typename T>
__global__ void __launch_bounds__(256) to_f32_kernel(const T* x, int64_t n, float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = to_f32<T>(x[i]);
}

// D[row] = sum_d dO[row][d] O'[row][d], one wave per row.
template <typename TO>
__global__ void __launch_bounds__(256) row_dot_kernel(const float* dout, const TO* ohp, int64_t rows, int d,
                                                      float* D) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float s = 0.0f;
  for (int c = lane; c < d; c += 64) s = __builtin_fmaf(dout[row * d + c], to_f32<TO>(ohp[row * d + c]), s);
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) s += __shfl_xor(s, k, 64);
  if (lane == 0) D[row] = s;
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

// ---- batched GEMM on the bf16 MFMA -----------------------------------------
//
// The products keep binary32 accuracy on the bf16 matrix instructions: an
// operand whose values are bf16 numbers (the dequantized NVFP4 Q^, K^, V^ --
// an E2M1 value times an E4M3 scale has at most 6 significant bits -- and dO
// given in bf16) goes in as it is; an fp32 operand (P^, dS, dO given in
// fp16) is split as x = hi + lo + r with hi = bf16(x), lo = bf16(x - hi),
// |r| <= 2^-17 |x|, and each product takes hi.hi + hi.lo + lo.hi (the lo.lo
// term is below 2^-16 of the product).  Products are exact in the MFMA and
// accumulate in fp32.

struct GemmArgs {
  const float* A;
  const float* B;
  float* C;
  int64_t M, N, K, lda, ldb, ldc, sA, sB, sC;
  int gA, gB;          // batch z reads A batch z / gA and B batch z / gB
  // causal structure (the score matrix is zero above the diagonal):
  // 2: K runs over keys (dS K^) -- the k loop stops after the tile's last query;
  // 3: M runs over keys, K over stacked query rows of Sq each (P^T dO, dS^T Q^)
  //    -- k slices whose queries all precede the tile's first key are skipped.
  int causal;
  int64_t Sq;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kGK = 32;   // k slice
constexpr int kGRow = kGK + 8;  // LDS row: 32 bf16 + 8 of padding (80 bytes)

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // finite values only
}

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

// One operand's slice: kGT rows (m or n) x kGK k, 16 values per thread.
// KC (k contiguous in memory, element (r, k) at X[r*ld + k]): thread t reads
// row t/8 + 32i, k 4(t%8)..+3.  RC (rows contiguous, element (r, k) at
// X[k*ld + r]): thread t reads rows 4(t%32)..+3 at k 4(t/32)+i and
// transposes in registers.
template <bool RC>
struct OpSlice {
  float4_t v[4];
  __device__ __forceinline__ void load(const float* X, int64_t ld, int64_t r0, int64_t rows, int64_t k0, int64_t kend) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!RC) {
        const int64_t r = r0 + t / 8 + 32 * i, k = k0 + 4 * (t % 8);
        v[i] = (r < rows && k < kend) ? *reinterpret_cast<const float4_t*>(X + r * ld + k) : float4_t{0, 0, 0, 0};
      } else {
        const int64_t r = r0 + 4 * (t % 32), k = k0 + 4 * (t / 32) + i;
        v[i] = (r < rows && k < kend) ? *reinterpret_cast<const float4_t*>(X + k * ld + r) : float4_t{0, 0, 0, 0};
      }
    }
  }
  template <bool SPLIT>
  __device__ __forceinline__ void store(uint16_t* hiS, uint16_t* loS) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4_t x;
      int r, k;
      if (!RC) {
        x = v[i];
        r = t / 8 + 32 * i;
        k = 4 * (t % 8);
      } else {
        x = float4_t{v[0][i], v[1][i], v[2][i], v[3][i]};  // row 4(t%32)+i, k 4(t/32)..+3
        r = 4 * (t % 32) + i;
        k = 4 * (t / 32);
      }
      uint2_t h, l;
      split4<SPLIT>(x, h, l);
      *reinterpret_cast<uint2_t*>(hiS + r * kGRow + k) = h;
      if (SPLIT) *reinterpret_cast<uint2_t*>(loS + r * kGRow + k) = l;
    }
  }
};

__device__ __forceinline__ float16_t mfma_bf16(const uint4_t& a, const uint4_t& b, const float16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// C[z] = op(A) op(B): op(A) is M x K (TA: A stored K x M), op(B) is K x N (TB:
// B stored N x K).  128 x 128 tile per workgroup (4 waves of 64 x 64, each
// 2 x 2 products of 32 x 32), 32-deep k slices through LDS; the next slice's
// loads are in flight while the current one computes.
template <bool TA, bool TB, bool SA, bool SB>
__global__ void __launch_bounds__(256) mgemm_kernel(GemmArgs g) {
  __shared__ uint16_t Ah[kGT * kGRow], Bh[kGT * kGRow];
  __shared__ uint16_t Al[SA ? kGT * kGRow : 1], Bl[SB ? kGT * kGRow : 1];
  const int64_t z = blockIdx.z;
  const float* A = g.A + (z / g.gA) * g.sA;
  const float* B = g.B + (z / g.gB) * g.sB;
  float* C = g.C + z * g.sC;
  const int64_t m0 = (int64_t)blockIdx.y * kGT, n0 = (int64_t)blockIdx.x * kGT;
  const int64_t kend = g.causal == 2 && m0 + kGT < g.K ? m0 + kGT : g.K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, hi = lane >> 5, r32 = lane & 31;
  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = float16_t{0};
  // first slice that is not all zero (mode 3: queries of the slice all before the tile's first key)
  auto skip = [&](int64_t k0) { return g.causal == 3 && (k0 % g.Sq) + kGK - 1 < m0; };
  OpSlice<TA> sa;      // A rows are m: contiguous along m when A is stored K x M
  OpSlice<!TB> sb;     // B rows are n: contiguous along n when B is stored K x N
  int64_t k0 = 0;
  while (k0 < kend && skip(k0)) k0 += kGK;
  if (k0 < kend) {
    sa.load(A, g.lda, m0, g.M, k0, kend);
    sb.load(B, g.ldb, n0, g.N, k0, kend);
  }
  while (k0 < kend) {
    __syncthreads();  // the previous slice's LDS reads are done
    sa.template store<SA>(Ah, Al);
    sb.template store<SB>(Bh, Bl);
    int64_t kn = k0 + kGK;
    while (kn < kend && skip(kn)) kn += kGK;
    if (kn < kend) {
      sa.load(A, g.lda, m0, g.M, kn, kend);
      sb.load(B, g.ldb, n0, g.N, kn, kend);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGK / 16; ++kk) {
      const int ko = 16 * kk + 8 * hi;
      uint4_t ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = (2 * wm + i) * 32 + r32, rb = (2 * wn + i) * 32 + r32;
        ah[i] = *reinterpret_cast<const uint4_t*>(Ah + ra * kGRow + ko);
        bh[i] = *reinterpret_cast<const uint4_t*>(Bh + rb * kGRow + ko);
        if (SA) al[i] = *reinterpret_cast<const uint4_t*>(Al + ra * kGRow + ko);
        if (SB) bl[i] = *reinterpret_cast<const uint4_t*>(Bl + rb * kGRow + ko);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = mfma_bf16(ah[i], bh[j], acc[i][j]);
          if (SB) acc[i][j] = mfma_bf16(ah[i], bl[j], acc[i][j]);
          if (SA) acc[i][j] = mfma_bf16(al[i], bh[j], acc[i][j]);
        }
    }
    k0 = kn;
  }
  // C layout of a 32 x 32 product: lane column r32, rows 8(v/4) + 4 hi + v%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + (2 * wn + j) * 32 + r32;
      if (col >= g.N) continue;
      const int64_t rb = m0 + (2 * wm + i) * 32 + 4 * hi;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = rb + 8 * (v / 4) + (v % 4);
        if (row < g.M) C[row * g.ldc + col] = acc[i][j][v];
      }
    }
}

template <bool TA, bool TB, bool SA, bool SB>
hipError_t gemm(const GemmArgs& g, int64_t batch, hipStream_t st) {
  const dim3 grid((unsigned)((g.N + kGT - 1) / kGT), (unsigned)((g.M + kGT - 1) / kGT), (unsigned)batch);
  hipLaunchKernelGGL((mgemm_kernel<TA, TB, SA, SB>), grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

// ---- scores, probabilities and dS in one pass -------------------------------
//
// One workgroup per 128 query rows (4 waves x 32) of a head, looping over the
// key tiles the rows see.  Per tile the waves compute S^T = K^ Q^T and
// dP^T = V^ dO^T on the bf16 MFMA (K^ and V^ rows fed in the permuted order
// that leaves each lane 16 consecutive keys of its query: one P block per
// lane), then the forward's tile-local P^ (the block scale from the block
// maximum, the tile maximum over kv_tile keys), P = 2^(x - lse2) and
// dS = s P (dP - D), and write P^ and dS.  Rows are written up to the end of
// the diagonal tile under the causal mask (the products read no further).

struct SdpArgs {
  const float *q, *k, *v, *dout, *D, *lse;
  float *Ph, *dS;
  int64_t H, G, Sq, Sk;
  int kv_tile, causal, single, nqt;
  float c, alpha;
};

__device__ __forceinline__ int sdp_krow(int r) { return (r & 3) | ((r >> 3) << 2) | (((r >> 2) & 1) << 4); }

__device__ __forceinline__ float sdp_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// 8 consecutive fp32 of a row -> 8 bf16 (hi, and lo when SPLIT) for an MFMA operand
template <bool SPLIT>
__device__ __forceinline__ void frag8(const float* p, bool ok, uint4_t& hi, uint4_t& lo) {
  const float4_t a = ok ? *reinterpret_cast<const float4_t*>(p) : float4_t{0, 0, 0, 0};
  const float4_t b = ok ? *reinterpret_cast<const float4_t*>(p + 4) : float4_t{0, 0, 0, 0};
  uint2_t ha, la, hb, lb;
  split4<SPLIT>(a, ha, la);
  split4<SPLIT>(b, hb, lb);
  hi = uint4_t{ha[0], ha[1], hb[0], hb[1]};
  lo = uint4_t{la[0], la[1], lb[0], lb[1]};
}

template <int D, bool SPLIT_DO>
__global__ void __launch_bounds__(256, 2) sdp_kernel(SdpArgs A) {
  constexpr int ROW = D + 8;  // bf16 per LDS row (16 bytes of padding)
  __shared__ uint16_t Ks[kGT * ROW], Vs[kGT * ROW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hi = lane >> 5, r32 = lane & 31;
  const int64_t BH = gridDim.x / A.nqt;
  const int64_t gi = blockIdx.x;
  const int64_t bh = gi % BH, qrank = gi / BH;
  const int qt = (int)(A.causal ? A.nqt - 1 - qrank : qrank);  // heaviest causal rows first
  const int64_t b = bh / A.H, h = bh - b * A.H;
  const int64_t bhk = b * (A.H / A.G) + h / A.G;
  const int64_t q = (int64_t)qt * kGT + 32 * wave + r32;
  const bool qok = q < A.Sq;
  const int64_t qidx = bh * A.Sq + (qok ? q : 0);
  // B operands (this lane's query, d = 16 s + 8 hi .. + 8): Q^ and dO
  uint4_t qf[D / 16], df[D / 16], dl[SPLIT_DO ? D / 16 : 1];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    uint4_t unused;
    frag8<false>(A.q + qidx * D + 16 * s + 8 * hi, qok, qf[s], unused);
    frag8<SPLIT_DO>(A.dout + qidx * D + 16 * s + 8 * hi, qok, df[s], dl[SPLIT_DO ? s : 0]);
  }
  const float lse2 = qok ? A.lse[qidx] * 1.4426950408889634f : 0.0f;
  const float Dq = qok ? A.D[qidx] : 0.0f;
  const int64_t qend = ((int64_t)qt + 1) * kGT;
  const int64_t kend = A.causal && qend < A.Sk ? qend : A.Sk;
  const int ntile = (int)((kend + kGT - 1) / kGT);
  const float* kb = A.k + bhk * A.Sk * D;
  const float* vb = A.v + bhk * A.Sk * D;
  const int krow = sdp_krow(r32);
  for (int t = 0; t < ntile; ++t) {
    const int64_t key0 = (int64_t)t * kGT;
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll 4
    for (int u = 0; u < kGT * D / 4 / 256; ++u) {
      const int f = threadIdx.x + 256 * u;
      const int r = f / (D / 4), c4 = f % (D / 4);
      const bool ok = key0 + r < A.Sk;
      const float4_t kx = ok ? *reinterpret_cast<const float4_t*>(kb + (key0 + r) * D + 4 * c4) : float4_t{0, 0, 0, 0};
      const float4_t vx = ok ? *reinterpret_cast<const float4_t*>(vb + (key0 + r) * D + 4 * c4) : float4_t{0, 0, 0, 0};
      uint2_t kh, vh, unused;
      split4<false>(kx, kh, unused);  // K^ and V^ are bf16 numbers: exact
      split4<false>(vx, vh, unused);
      *reinterpret_cast<uint2_t*>(Ks + r * ROW + 4 * c4) = kh;
      *reinterpret_cast<uint2_t*>(Vs + r * ROW + 4 * c4) = vh;
    }
    __syncthreads();
    // S^T for the tile's four 32-key subtiles
    float16_t sacc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      sacc[g] = float16_t{0};
      const uint16_t* ka = Ks + (32 * g + krow) * ROW + 8 * hi;
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        sacc[g] = mfma_bf16(*reinterpret_cast<const uint4_t*>(ka + 16 * s), qf[s], sacc[g]);
    }
    // x = fl32(S c) on visible keys, block and tile maxima
    float bmax[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float m = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t key = key0 + 32 * g + 16 * hi + i;
        const bool vis = key < A.Sk && (!A.causal || key <= q);
        sacc[g][i] = vis ? sacc[g][i] * A.c : -__builtin_inff();
        m = __builtin_fmaxf(m, sacc[g][i]);
      }
      bmax[g] = m;
    }
    float tmv[4];
    if (A.kv_tile == 128) {
      float m = __builtin_fmaxf(__builtin_fmaxf(bmax[0], bmax[1]), __builtin_fmaxf(bmax[2], bmax[3]));
      m = __builtin_fmaxf(m, sdp_xor32(m));
      tmv[0] = tmv[1] = tmv[2] = tmv[3] = m;
    } else {
      float m0 = __builtin_fmaxf(bmax[0], bmax[1]), m1 = __builtin_fmaxf(bmax[2], bmax[3]);
      m0 = __builtin_fmaxf(m0, sdp_xor32(m0));
      m1 = __builtin_fmaxf(m1, sdp_xor32(m1));
      tmv[0] = tmv[1] = m0;
      tmv[2] = tmv[3] = m1;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t kb0 = key0 + 32 * g + 16 * hi;  // this lane's P block
      // dP^T of the subtile
      float16_t dp = float16_t{0};
      const uint16_t* va = Vs + (32 * g + krow) * ROW + 8 * hi;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const uint4_t a = *reinterpret_cast<const uint4_t*>(va + 16 * s);
        dp = mfma_bf16(a, df[s], dp);
        if (SPLIT_DO) dp = mfma_bf16(a, dl[s], dp);
      }
      float pv[16], ph[16];
      const float tm = tmv[g];
      if (bmax[g] == -__builtin_inff()) {
#pragma unroll
        for (int i = 0; i < 16; ++i) pv[i] = ph[i] = 0.0f;
      } else {
        const float emax = __builtin_amdgcn_exp2f(bmax[g] - tm);
        const uint32_t byte = f32_to_e4m3(A.single ? div6_rn(emax) : emax * 448.0f);
        const float2_t fs = A.single ? kTrainP.one[byte] : kTrainP.two[byte];
        const float w = __builtin_amdgcn_exp2f(tm - lse2) * (A.single ? 1.0f : 1.0f / 2688.0f);
        float tq[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) tq[i] = __builtin_amdgcn_exp2f(sacc[g][i] - tm) * fs[0];  // masked: 0
        uint32_t cw[2] = {0u, 0u};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          cw[hh] = cvt_pk_fp4<0>(cw[hh], tq[8 * hh + 0], tq[8 * hh + 1]);
          cw[hh] = cvt_pk_fp4<1>(cw[hh], tq[8 * hh + 2], tq[8 * hh + 3]);
          cw[hh] = cvt_pk_fp4<2>(cw[hh], tq[8 * hh + 4], tq[8 * hh + 5]);
          cw[hh] = cvt_pk_fp4<3>(cw[hh], tq[8 * hh + 6], tq[8 * hh + 7]);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float2_t a0 = cvt_pk_f32_fp4<0>(cw[hh]), a1 = cvt_pk_f32_fp4<1>(cw[hh]);
          const float2_t a2 = cvt_pk_f32_fp4<2>(cw[hh]), a3 = cvt_pk_f32_fp4<3>(cw[hh]);
          const float cv[8] = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
#pragma unroll
          for (int i = 0; i < 8; ++i) ph[8 * hh + i] = cv[i] * fs[1] * w;  // code value times s2 is exact
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(sacc[g][i] - lse2);
      }
      if (qok && kb0 < A.Sk) {
        float* php = A.Ph + qidx * A.Sk + kb0;
        float* dsp = A.dS + qidx * A.Sk + kb0;
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          *reinterpret_cast<float4_t*>(php + i) = float4_t{ph[i], ph[i + 1], ph[i + 2], ph[i + 3]};
          *reinterpret_cast<float4_t*>(dsp + i) =
              float4_t{A.alpha * pv[i] * (dp[i] - Dq), A.alpha * pv[i + 1] * (dp[i + 1] - Dq),
                       A.alpha * pv[i + 2] * (dp[i + 2] - Dq), A.alpha * pv[i + 3] * (dp[i + 3] - Dq)};
        }
      }
    }
  }
}

}  // namespace fp4dev

using namespace fp4dev;

size_t fp4i_attn_bwd_workspace(const AttnBwdLaunch& L) {
  auto a = [](size_t n) { return (n + 255) & ~(size_t)255; };
  const size_t nq = (size_t)(L.B * L.H * L.Sq), nk = (size_t)(L.B * L.Hkv * L.Sk);
  return a(nq * L.d * 4) * 2 + a(nk * L.d * 4) * 2 + a(nq * 4) + a(nq * (size_t)L.Sk * 4) * 2;
}

hipError_t fp4i_launch_attn_bwd(const AttnBwdLaunch& L, hipStream_t st) {
  auto a = [](size_t n) { return (n + 255) & ~(size_t)255; };
  const int64_t B = L.B, H = L.H, Hkv = L.Hkv, Sq = L.Sq, Sk = L.Sk, d = L.d, G = H / Hkv;
  const size_t nq = (size_t)(B * H * Sq), nk = (size_t)(B * Hkv * Sk);
  const bool fp16_do = L.dtype == 1;  // dO in fp16 is not a bf16 number: split it
  char* w = (char*)L.ws;
  float* qh = (float*)w; w += a(nq * d * 4);
  float* dof = (float*)w; w += a(nq * d * 4);
  float* kh = (float*)w; w += a(nk * d * 4);
  float* vh = (float*)w; w += a(nk * d * 4);
  float* Dv = (float*)w; w += a(nq * 4);
  float* Sb = (float*)w; w += a(nq * (size_t)Sk * 4);
  float* Ph = (float*)w;
  auto blocks = [](int64_t n) { return dim3((unsigned)((n + 255) / 256)); };
  // operands
  hipLaunchKernelGGL(dequant_rows_kernel, blocks((int64_t)nq * d / 8), dim3(256), 0, st, L.qc, L.qs, (int64_t)nq,
                     (int)d, qh);
  hipLaunchKernelGGL(dequant_rows_kernel, blocks((int64_t)nk * d / 8), dim3(256), 0, st, L.kc, L.ks, (int64_t)nk,
                     (int)d, kh);
  hipLaunchKernelGGL(dequant_cols_kernel, blocks((int64_t)nk / 2 * d), dim3(256), 0, st, L.vc, L.vs, (int64_t)nk,
                     (int)d, vh);
  if (L.dtype == 1)
    hipLaunchKernelGGL(to_f32_kernel<half_t>, blocks((int64_t)nq * d), dim3(256), 0, st, (const half_t*)L.dout,
                       (int64_t)nq * d, dof);
  else
    hipLaunchKernelGGL(to_f32_kernel<uint16_t>, blocks((int64_t)nq * d), dim3(256), 0, st, (const uint16_t*)L.dout,
                       (int64_t)nq * d, dof);
  const dim3 rd((unsigned)((nq + 3) / 4));
  if (L.hp_dtype == 2) hipLaunchKernelGGL(row_dot_kernel<float>, rd, dim3(256), 0, st, dof, (const float*)L.out_hp, (int64_t)nq, (int)d, Dv);
  else if (L.hp_dtype == 1) hipLaunchKernelGGL(row_dot_kernel<half_t>, rd, dim3(256), 0, st, dof, (const half_t*)L.out_hp, (int64_t)nq, (int)d, Dv);
  else hipLaunchKernelGGL(row_dot_kernel<uint16_t>, rd, dim3(256), 0, st, dof, (const uint16_t*)L.out_hp, (int64_t)nq, (int)d, Dv);
  // P^ and dS = s P (dO V^T - D) from the scores, in one pass
  SdpArgs sa;
  sa.q = qh; sa.k = kh; sa.v = vh; sa.dout = dof; sa.D = Dv; sa.lse = L.lse;
  sa.Ph = Ph; sa.dS = Sb;
  sa.H = H; sa.G = G; sa.Sq = Sq; sa.Sk = Sk;
  sa.kv_tile = L.kv_tile; sa.causal = L.causal; sa.single = L.single;
  sa.nqt = (int)((Sq + kGT - 1) / kGT);
  sa.c = L.c;
  sa.alpha = L.c * 0.69314718055994531f;
  const dim3 sgrid((unsigned)(B * H * sa.nqt));
  if (d == 128) {
    if (fp16_do) hipLaunchKernelGGL((sdp_kernel<128, true>), sgrid, dim3(256), 0, st, sa);
    else hipLaunchKernelGGL((sdp_kernel<128, false>), sgrid, dim3(256), 0, st, sa);
  } else {
    if (fp16_do) hipLaunchKernelGGL((sdp_kernel<64, true>), sgrid, dim3(256), 0, st, sa);
    else hipLaunchKernelGGL((sdp_kernel<64, false>), sgrid, dim3(256), 0, st, sa);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dV = P^T dO over the G query heads of each kv head
  GemmArgs g{};
  g.A = Ph; g.lda = Sk; g.sA = G * Sq * Sk; g.gA = 1;
  g.B = dof; g.ldb = d; g.sB = G * Sq * d; g.gB = 1;
  g.C = L.dv; g.ldc = d; g.sC = Sk * d;
  g.M = Sk; g.N = d; g.K = G * Sq;
  g.causal = L.causal ? 3 : 0;
  g.Sq = Sq;
  if ((e = (fp16_do ? gemm<true, false, true, true>(g, B * Hkv, st) : gemm<true, false, true, false>(g, B * Hkv, st))) != hipSuccess) return e;
  // dQ = dS K^
  g = GemmArgs{};
  g.A = Sb; g.lda = Sk; g.sA = Sq * Sk; g.gA = 1;
  g.B = kh; g.ldb = d; g.sB = Sk * d; g.gB = (int)G;
  g.C = L.dq; g.ldc = d; g.sC = Sq * d;
  g.M = Sq; g.N = d; g.K = Sk;
  g.causal = L.causal ? 2 : 0;
  if ((e = gemm<false, false, true, false>(g, B * H, st)) != hipSuccess) return e;
  // dK = dS^T Q^ over the G query heads of each kv head
  g = GemmArgs{};
  g.A = Sb; g.lda = Sk; g.sA = G * Sq * Sk; g.gA = 1;
  g.B = qh; g.ldb = d; g.sB = G * Sq * d; g.gB = 1;
  g.C = L.dk; g.ldc = d; g.sC = Sk * d;
  g.M = Sk; g.N = d; g.K = G * Sq;
  g.causal = L.causal ? 3 : 0;
  g.Sq = Sq;
  return gemm<true, false, true, false>(g, B * Hkv, st);
}

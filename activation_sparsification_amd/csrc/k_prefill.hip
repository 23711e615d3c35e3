// Prefill GEMM on the matrix cores: y[t][n_out] = nu * (A W^T) + eta * rowsum.
//
// A is the pruned activation; W is the layer's own [n_out][k] weight (both
// operands contiguous along k, which is how the matrix-core fragments want
// them).  For 2:4 the pruning pass has packed A to its kept half plus one
// nibble of in-block positions per block, and the gfx950 sparse MFMA
// (v_smfmac_f32_16x16x64) skips the pruned products -- the 2:4 scheme of
// "Accelerating Transformer training and inference with 2:4 sparsity and
// Squared-ReLU" s2.1/s3.1 on CDNA4's own instruction.  Other n:m patterns
// run dense MFMA (v_mfma_f32_16x16x32) on the masked rows.
//
// Fragment layouts (gfx950, lane l, g = l / 16):
//   smfmac A: row l%16, 8 packed values = logical k [16g, 16g+16) of the
//             64-wide step, position bits from the 16-bit half given by abid;
//   smfmac B: column l%16, k = 8g..8g+7 then 32+8g..32+8g+7;
//   mfma   A: row l%16, k = 8g..8g+7;  B: column l%16, k = 8g..8g+7;
//   D:        column l%16, rows 4g..4g+3.
//
// Tiling: BM x BN per workgroup, four waves in a 2 x 2 grid, k in steps of
// 64 (logical).  Global tiles go through registers into a double-buffered
// LDS stage (rows padded by 16 bytes against bank conflicts).  Workgroups
// are ordered so that one XCD (each has its own L2) works through all the
// token tiles of one weight tile before moving on.
#include "spa_common.h"
#include "spa_launch.h"

namespace spa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Frag;
template <> struct Frag<SPA_BF16> { using V8 = bf16x8; using V16 = bf16x16; };
template <> struct Frag<SPA_F16> { using V8 = f16x8; using V16 = f16x16; };

template <int DT>
__device__ __forceinline__ f32x4 smfmac(const typename Frag<DT>::V8& a, const typename Frag<DT>::V16& b, f32x4 c,
                                        int idx) {
  if constexpr (DT == SPA_BF16) return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a, b, c, idx, 0, 0);
  else return __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, c, idx, 0, 0);
}
template <int DT>
__device__ __forceinline__ f32x4 mfma(const typename Frag<DT>::V8& a, const typename Frag<DT>::V8& b, f32x4 c) {
  if constexpr (DT == SPA_BF16) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <class V>
__device__ __forceinline__ V as_vec(const uint4& u) { return __builtin_bit_cast(V, u); }

// SPARSE: A row holds 32 packed halves (64 B) + 4 uint16 meta per 64-wide step.
// DENSE : A row holds 64 halves (128 B).
template <int DT, bool SPARSE, int BM, int BN>
__global__ void __launch_bounds__(256) k_gemm(PrefillArgs p) {
  constexpr int BK = 64;
  constexpr int AH = SPARSE ? 32 : 64;          // A halves per row per step
  constexpr int APAD = AH + 8;                  // padded LDS row (halves)
  constexpr int BPAD = BK + 8;
  constexpr int WM = BM / 2, WN = BN / 2;       // wave tile
  constexpr int FM = WM / 16, FN = WN / 16;     // fragments per wave
  constexpr int A_SEGS = BM * AH / 8;           // 16-byte segments per A tile
  constexpr int B_SEGS = BN * BK / 8;
  constexpr int A_PER = (A_SEGS + 255) / 256;
  constexpr int B_PER = (B_SEGS + 255) / 256;
  constexpr int A_SEG_ROW = AH / 8, B_SEG_ROW = BK / 8;
  using V8 = typename Frag<DT>::V8;
  using V16 = typename Frag<DT>::V16;

  __shared__ __attribute__((aligned(16))) uint16_t s_a[2][BM][APAD];
  __shared__ __attribute__((aligned(16))) uint16_t s_b[2][BN][BPAD];
  __shared__ uint16_t s_m[2][SPARSE ? BM : 1][4];

  const int T = p.t, K = p.k, N = p.n_out;
  const int tiles_m = (T + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a contiguous
  // run of tile indices, token tiles fastest.
  int bid = blockIdx.x;
  const int per_xcd = total / 8;
  if (bid < per_xcd * 8) bid = (bid % 8) * per_xcd + bid / 8;
  const int tm = bid % tiles_m, tn = bid / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int wm0 = (wv >> 1) * WM, wn0 = (wv & 1) * WN;

  const uint16_t* A = static_cast<const uint16_t*>(p.a_vals);
  const uint16_t* W = static_cast<const uint16_t*>(p.w);
  const int a_row_halves = SPARSE ? K / 2 : K;

  uint4 ra[A_PER], rb[B_PER];
  uint2 rm;
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int s = threadIdx.x + 256 * i;
      const int r = s / A_SEG_ROW, c = s % A_SEG_ROW;
      const int row = m0 + r;
      if (s < A_SEGS && row < T)
        ra[i] = *reinterpret_cast<const uint4*>(A + (size_t)row * a_row_halves + (size_t)kt * AH + c * 8);
      else
        ra[i] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int s = threadIdx.x + 256 * i;
      const int r = s / B_SEG_ROW, c = s % B_SEG_ROW;
      const int row = n0 + r;
      if (s < B_SEGS && row < N)
        rb[i] = *reinterpret_cast<const uint4*>(W + (size_t)row * K + (size_t)kt * BK + c * 8);
      else
        rb[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    if constexpr (SPARSE) {
      const int row = m0 + (int)threadIdx.x;
      if ((int)threadIdx.x < BM && row < T)
        rm = *reinterpret_cast<const uint2*>(p.a_meta + (size_t)row * (K / 16) + (size_t)kt * 4);
      else
        rm = make_uint2(0x44444444u, 0x44444444u);  // positions (0,1): valid, multiplies zeros
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int s = threadIdx.x + 256 * i;
      if (s < A_SEGS) {
        const int r = s / A_SEG_ROW, c = s % A_SEG_ROW;
        *reinterpret_cast<uint4*>(&s_a[buf][r][c * 8]) = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int s = threadIdx.x + 256 * i;
      if (s < B_SEGS) {
        const int r = s / B_SEG_ROW, c = s % B_SEG_ROW;
        *reinterpret_cast<uint4*>(&s_b[buf][r][c * 8]) = rb[i];
      }
    }
    if constexpr (SPARSE) {
      if ((int)threadIdx.x < BM) *reinterpret_cast<uint2*>(&s_m[buf][threadIdx.x][0]) = rm;
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    if constexpr (SPARSE) {
      V16 bf[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint16_t* br = &s_b[buf][wn0 + j * 16 + l16][0];
        const uint4 lo = *reinterpret_cast<const uint4*>(br + 8 * g);
        const uint4 hi = *reinterpret_cast<const uint4*>(br + 32 + 8 * g);
        const uint4 both[2] = {lo, hi};
        bf[j] = __builtin_bit_cast(V16, both);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm0 + i * 16 + l16;
        const V8 af = as_vec<V8>(*reinterpret_cast<const uint4*>(&s_a[buf][r][8 * g]));
        const int idx = (int)s_m[buf][r][g];
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = smfmac<DT>(af, bf[j], acc[i][j], idx);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        V8 bf[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bf[j] = as_vec<V8>(*reinterpret_cast<const uint4*>(&s_b[buf][wn0 + j * 16 + l16][32 * s + 8 * g]));
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const V8 af = as_vec<V8>(*reinterpret_cast<const uint4*>(&s_a[buf][wm0 + i * 16 + l16][32 * s + 8 * g]));
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma<DT>(af, bf[j], acc[i][j]);
        }
      }
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: y = nu_i * acc + eta_i * rowsum_j
  uint16_t* Y = static_cast<uint16_t*>(p.y);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm0 + i * 16 + 4 * g + r;
      if (row >= T) continue;
      const float nu = p.nu ? p.nu[row] : 1.f;
      const float eta = p.eta ? p.eta[row] : 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn0 + j * 16 + l16;
        if (col < N) {
          float v = nu * acc[i][j][r];
          if (p.eta) v += eta * p.row_sum[col];
          Y[(size_t)row * N + col] = (uint16_t)from_f32<DT>(v);
        }
      }
    }
  }
}

template <int DT, bool SPARSE>
static hipError_t gemm_launch(const PrefillArgs& a, hipStream_t st) {
  constexpr int BM = 256, BN = 256;
  const int tiles = ((a.t + BM - 1) / BM) * ((a.n_out + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm<DT, SPARSE, BM, BN>), dim3(tiles), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, const PrefillArgs& a, hipStream_t st) {
  if (a.t == 0) return hipSuccess;
  if (dtype == SPA_F16) return a.sparse24 ? gemm_launch<SPA_F16, true>(a, st) : gemm_launch<SPA_F16, false>(a, st);
  return a.sparse24 ? gemm_launch<SPA_BF16, true>(a, st) : gemm_launch<SPA_BF16, false>(a, st);
}

}  // namespace spa

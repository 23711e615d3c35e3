// Prefill GEMM on the matrix cores: y[t][n_out] = nu * (A W^T) + eta * rowsum.
//
// A is the pruned activation; W is the layer's own [n_out][k] weight (both
// operands contiguous along k, which is how the matrix-core fragments want
// them).  For 2:4 the pruning pass has packed A to its kept half plus one
// nibble of in-block positions per block, and the gfx950 sparse MFMA
// (v_smfmac_f32_32x32x32) skips the pruned products -- the 2:4 scheme of
// "Accelerating Transformer training and inference with 2:4 sparsity and
// Squared-ReLU" s2.1/s3.1 on CDNA4's own instruction.  Other n:m patterns
// run dense MFMA (v_mfma_f32_32x32x16) on the masked rows.
//
// Fragment layouts (gfx950, lane l, l32 = l % 32, g = l / 32):
//   smfmac A: row l32, 8 packed values = logical k [16g, 16g+16) of each
//             32-wide half step, position bits from the 16-bit half of the
//             index operand;
//   smfmac B: column l32, k = 8g..8g+7 then 16+8g..16+8g+7 (per half step);
//   mfma   A: row l32, k = 8g..8g+7;  B: column l32, same k;
//   D:        register r holds row 8(r/4) + 4g + r%4, column l32.
//
// Both kernels stream 64-wide k steps through a three-stage LDS ring filled
// by direct global->LDS loads (no register staging), with two or more waves
// per SIMD (so one wave's matrix instructions cover another's LDS reads):
// 8 waves for the dense GEMM; 8, 12 or 16 for the 2:4 GEMM (see k_gemm24).
// Workgroups are ordered so that one XCD (each has its own L2) works through
// a block of token tiles by weight tiles before moving on.
#include "spa_common.h"
#include "spa_launch.h"

namespace spa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int DT> struct Frag;
template <> struct Frag<SPA_BF16> { using V8 = bf16x8; using V16 = bf16x16; };
template <> struct Frag<SPA_F16> { using V8 = f16x8; using V16 = f16x16; };

template <class V>
__device__ __forceinline__ V as_vec(const uint4& u) { return __builtin_bit_cast(V, u); }

// Two 16-byte chunks as one 16-element operand (lo = elements 0..7).
template <int DT>
__device__ __forceinline__ typename Frag<DT>::V16 cat16(const uint4& lo, const uint4& hi) {
  const uint4 both[2] = {lo, hi};
  return __builtin_bit_cast(typename Frag<DT>::V16, both);
}

template <int DT>
__device__ __forceinline__ f32x16 smfmac32(const typename Frag<DT>::V8& a, const typename Frag<DT>::V16& b, f32x16 c,
                                           int idx) {
  if constexpr (DT == SPA_BF16) return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, b, c, idx, 0, 0);
  else return __builtin_amdgcn_smfmac_f32_32x32x32_f16(a, b, c, idx, 0, 0);
}
template <int DT>
__device__ __forceinline__ f32x16 mfma32(const typename Frag<DT>::V8& a, const typename Frag<DT>::V8& b, f32x16 c) {
  if constexpr (DT == SPA_BF16) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// XCD-aware tile order: workgroup b runs on XCD b % 8; each XCD gets a
// contiguous run of tile indices.  Tiles are numbered in groups of (up to) 8
// token tiles times every weight tile, token tiles fastest, so an XCD's run
// is a block of at most 8 token tiles by a few weight tiles: its L2 serves
// each weight tile to those token tiles and each token tile to those weight
// tiles (instead of every XCD reading every token tile).
__device__ __forceinline__ void xcd_tile(int T, int N, int BM, int BN, int& tm, int& tn) {
  constexpr int GM = 8;
  const int tiles_m = (T + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  int bid = blockIdx.x;
  const int per_xcd = total / 8;
  if (bid < per_xcd * 8) bid = (bid % 8) * per_xcd + bid / 8;
  const int group = bid / (GM * tiles_n);
  const int m_first = group * GM;
  const int gm = min(tiles_m - m_first, GM);
  const int r = bid - group * GM * tiles_n;
  tm = m_first + r % gm;
  tn = r / gm;
}

// Epilogue operands of one tile (BM rows, BN columns): each thread fetches at
// most one nu, one eta and one row sum when the workgroup starts, holds them
// in registers across the main loop and parks them in LDS at the end.
template <int BM, int BN>
struct TileScalars {
  float nu, eta, rs;
  __device__ __forceinline__ void fetch(const PrefillArgs& p, int m0, int n0) {
    const int i = threadIdx.x;
    const int row = min(m0 + (i & (BM - 1)), p.t - 1);
    nu = (p.nu && i < BM) ? p.nu[row] : 1.f;
    eta = (p.eta && i < BM) ? p.eta[row] : 0.f;
    rs = (p.eta && i < BN) ? p.row_sum[min(n0 + i, p.n_out - 1)] : 0.f;
  }
  __device__ __forceinline__ void park(float* s_nu, float* s_eta, float* s_rs) const {
    const int i = threadIdx.x;
    if (i < BM) {
      s_nu[i] = nu;
      s_eta[i] = eta;
    }
    if (i < BN) s_rs[i] = rs;
  }
};

// y = nu_i * acc + eta_i * rowsum_j for a wave's FM x FN fragments of 32 x 32
// at tile-relative (r0, c0) of the tile that starts at (m0, n0), written
// through LDS: the wave stores its (FM*32) x (FN*32) block of 16-bit results
// row-major into `st` (its own region of the freed operand ring), then writes
// whole rows back as 16-byte pieces (eight of the fragment layout's two-byte
// stores become one).  Rows past t are dropped;
// columns past n_out (or any n_out not a multiple of 8) fall back to element
// stores.
// With a column scale s_cs (the FP8 GEMM's weight-row scales) the value is
// nu_i * cs_j * acc + eta_i * rs_j.
template <int DT, int FM, int FN, bool CS = false>
__device__ __forceinline__ void store_tile_lds(const PrefillArgs& p, const f32x16 (&acc)[FM][FN], int m0, int n0,
                                               int r0, int c0, int g, int l32, int lane, const float* s_nu,
                                               const float* s_eta, const float* s_rs, uint16_t* st,
                                               const float* s_cs = nullptr) {
  constexpr int W = FN * 32, H = FM * 32, GPR = W / 8, RPI = 64 / GPR;
  static_assert(64 % GPR == 0 && H % RPI == 0, "whole 16-byte groups per row");
  float rs[FN], cs[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    rs[j] = s_rs[c0 + 32 * j + l32];
    if constexpr (CS) cs[j] = s_cs[c0 + 32 * j + l32];
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lr = 32 * i + 8 * (r / 4) + 4 * g + (r % 4);
      const float nu = s_nu[r0 + lr], eta = s_eta[r0 + lr];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        float v;
        if constexpr (CS) v = nu * cs[j] * acc[i][j][r] + eta * rs[j];
        else v = nu * acc[i][j][r] + eta * rs[j];
        st[lr * W + 32 * j + l32] = (uint16_t)from_f32<DT>(v);
      }
    }
  }
  // the wave's LDS writes are complete before its reads (one wave, in order)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint16_t* Y = static_cast<uint16_t*>(p.y);
  const int N = p.n_out;
  const bool whole = N % 8 == 0;
#pragma unroll
  for (int q = 0; q < H / RPI; ++q) {
    const int rr = q * RPI + lane / GPR, gc = lane % GPR;
    const int row = m0 + r0 + rr, col = n0 + c0 + gc * 8;
    if (row >= p.t) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(st + rr * W + gc * 8);
    uint16_t* dst = Y + (size_t)row * N + col;
    if (whole && col < N) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < N) dst[e] = (uint16_t)(wd[e / 2] >> (16 * (e % 2)));
    }
  }
}

// ---------------------------------------------------------------------------
// 2:4 smfmac GEMM.  The pruning pass stores the packed activations and their
// position words step-major (per 64-channel step: rows padded to t_pad, 64 B
// of packed values and 8 B of position words per row), so a 256-row tile of
// one step is one contiguous run.  BM = BN = 256; NW = 8 waves in a 2 x 4
// grid of 128 x 64 (4 x 2 fragments of 32 x 32), or NW = 16 in a 4 x 4 grid
// of 64 x 64 (2 x 2 fragments).  With 8 waves every wave issues seven direct
// loads per step (two 1 KB runs of packed values, four 1 KB groups of weight
// rows, one 256 B run of position words); with 16, four (waves 0-7) or three.
// Waiting for vmcnt <= that count therefore means "the older of the two steps
// in flight has landed".
//
// Each stage lives in its own __shared__ arrays.  Rows are unpadded; 16-byte
// chunks are XOR-swizzled against bank conflicts: chunk c of activation row r
// sits at c ^ ((r >> 2) & 3), of weight row r at c ^ ((r >> 1) & 7).  Weight
// rows past n_out re-read the last row; padded activation rows hold whatever
// the workspace held.  Neither reaches y: outputs are stored for rows < t and
// columns < n_out only, and no row's result depends on another row.
// ---------------------------------------------------------------------------
template <int DT, int NW>
__global__ void __launch_bounds__(NW * 64, 1) k_gemm24(PrefillArgs p) {
  static_assert(NW == 8 || NW == 12 || NW == 16, "8 waves of 128 x 64, or 12 or 16 of 64 x 64");
  constexpr int BM = 256, BN = NW == 12 ? 192 : 256;
  constexpr int WM = NW == 8 ? 128 : 64, WN = 64, FM = WM / 32, FN = 2;
  constexpr int WC = BN / WN;                              // wave columns
  using V8 = typename Frag<DT>::V8;
  using V16 = typename Frag<DT>::V16;
  // stage = packed activations (BM x 64 B) followed by their position words
  // (BM x 8 B); three stages of each operand, back to back
  constexpr int AST = BM * 72, BST = BN * 128;            // bytes per stage
  __shared__ __attribute__((aligned(1024))) unsigned char sA[3 * AST];
  __shared__ __attribute__((aligned(1024))) unsigned char sB[3 * BST];
  __shared__ float s_nu[BM], s_eta[BM], s_rs[BN];

  const int K = p.k, N = p.n_out, TP = p.t_pad;
  int tm, tn;
  xcd_tile(p.t, p.col1 - p.col0, BM, BN, tm, tn);
  const int m0 = tm * BM, n0 = p.col0 + tn * BN;
  TileScalars<BM, BN> ts;
  ts.fetch(p, m0, n0);

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int wm0 = (wv / WC) * WM, wn0 = (wv % WC) * WN;

  // ---- direct-load sources: uniform per-step bases + 32-bit lane offsets ----
  const char* baseA = static_cast<const char*>(p.a_vals) + (size_t)m0 * 64;
  const char* baseM = reinterpret_cast<const char*>(p.a_meta) + (size_t)m0 * 8;
  const char* baseW = static_cast<const char*>(p.w) + (size_t)n0 * K * 2;
  const size_t stepA = (size_t)TP * 64, stepM = (size_t)TP * 8;
  // Per step, 8 waves: wave wv loads activation runs 2 wv, 2 wv + 1 (LDS slot
  // s of run r holds row 16 r + s/4), weight groups h = 0..3 (slot s of group
  // h holds row 8 (4 wv + h) + s/8) and the position words of rows 32 wv ..
  // +31.  16 waves: activation run wv, weight groups 2 wv, 2 wv + 1, and waves
  // 0-7 the position words as above.  12 waves (192 columns): activation run
  // wv and, for waves 0-3, run 12 + wv; weight groups 2 wv, 2 wv + 1; waves
  // 0-7 the position words.
  constexpr int NA = NW == 16 ? 1 : 2, NB = NW == 8 ? 4 : 2;
  const bool loads_m = NW == 8 || wv < 8;                 // wave-uniform
  const bool loads_a2 = NW != 12 || wv < 4;               // the second activation run
  int runA[NA];
#pragma unroll
  for (int h = 0; h < NA; ++h) runA[h] = NW == 8 ? 2 * wv + h : h == 0 ? wv : 12 + wv;
  uint32_t offA[NA], offB[NB];
#pragma unroll
  for (int h = 0; h < NA; ++h) {
    const int ra = 16 * runA[h] + (lane >> 2);
    offA[h] = (uint32_t)(ra * 64 + (((lane & 3) ^ ((ra >> 2) & 3)) * 16));
  }
#pragma unroll
  for (int h = 0; h < NB; ++h) {
    const int r = 8 * (NB * wv + h) + (lane >> 3);
    const int rr = min(n0 + r, N - 1) - n0;
    offB[h] = (uint32_t)rr * (uint32_t)K * 2u + (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) * 16);
  }
  const uint32_t offM = (uint32_t)(((wv & 7) * 64 + lane) * 4);
  const uint32_t ldsA0 = lds_addr(sA), ldsB0 = lds_addr(sB);

  // ---- LDS fragment offsets (bytes); the swizzle terms do not depend on i or j ----
  const int qa = (l32 >> 2) & 3, qb = (l32 >> 1) & 7;
  const int rowA = wm0 + l32, rowB = wn0 + l32;
  int ldsA[2], ldsBlo[2], ldsBhi[2], ldsM[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    ldsA[s] = rowA * 64 + (((2 * s + g) ^ qa) * 16);
    ldsBlo[s] = rowB * 128 + (((4 * s + g) ^ qb) * 16);
    ldsBhi[s] = rowB * 128 + (((4 * s + 2 + g) ^ qb) * 16);
    ldsM[s] = BM * 64 + rowA * 8 + (2 * s + g) * 2;
  }

#define SPA_ISSUE24(KT, ST)                                                              \
  do {                                                                                   \
    const char* a_ = baseA + (size_t)(KT) * stepA;                                       \
    const char* w_ = baseW + (size_t)(KT) * 128;                                         \
    const uint32_t la_ = ldsA0 + (ST) * AST, lb_ = ldsB0 + (ST) * BST + wv * (NB * 1024); \
    _Pragma("unroll") for (int h = 0; h < NA; ++h)                                       \
      if (h == 0 || loads_a2) lds_dma16(a_, offA[h], la_ + runA[h] * 1024);             \
    _Pragma("unroll") for (int h = 0; h < NB; ++h) lds_dma16(w_, offB[h], lb_ + h * 1024); \
    if (loads_m)                                                                         \
      lds_dma4(baseM + (size_t)(KT) * stepM, offM, ldsA0 + (ST) * AST + BM * 64 + (wv & 7) * 256); \
  } while (0)
  // loads per step: 7 for 8 waves; 4 (waves 0-7) or 3 for 16 waves; 5 (waves
  // 0-3), 4 (waves 4-7) or 3 for 12 waves
#define SPA_WAIT24(COND)                                                                 \
  do {                                                                                   \
    if constexpr (NW == 8) wait_vm<7>(COND);                                             \
    else if (NW == 12 && loads_a2) wait_vm<5>(COND);                                     \
    else if (loads_m) wait_vm<4>(COND);                                                  \
    else wait_vm<3>(COND);                                                               \
  } while (0)

  // fragments of one 32-wide half step, two register sets (set 0: first
  // half of a step, set 1: second half)
  V16 bf[2][FN];
  V8 af[2][FM];
  int ix[2][FM];
#define SPA_READ24(ST, S)                                                                \
  do {                                                                                   \
    const unsigned char* a_ = sA + (ST) * AST;                                           \
    const unsigned char* b_ = sB + (ST) * BST;                                           \
    _Pragma("unroll") for (int j = 0; j < FN; ++j)                                       \
      bf[S][j] = cat16<DT>(*reinterpret_cast<const uint4*>(b_ + ldsBlo[S] + j * 4096),   \
                           *reinterpret_cast<const uint4*>(b_ + ldsBhi[S] + j * 4096));  \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                     \
      af[S][i] = as_vec<V8>(*reinterpret_cast<const uint4*>(a_ + ldsA[S] + i * 2048));   \
      ix[S][i] = (int)*reinterpret_cast<const uint16_t*>(a_ + ldsM[S] + i * 256);        \
    }                                                                                    \
  } while (0)
#define SPA_MMA24(S)                                                                     \
  do {                                                                                   \
    _Pragma("unroll") for (int i = 0; i < FM; ++i)                                       \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                     \
        acc[i][j] = smfmac32<DT>(af[S][i], bf[S][j], acc[i][j], ix[S][i]);               \
  } while (0)

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Step kt lives in stage kt % 3.  Barrier B_kt sits between the two halves
  // of step kt-1's products: before it, every wave has read all of step kt-1
  // (so that stage is refilled with step kt+2 right after it) and waited for
  // its own copies of step kt; after it, the wave reads step kt's first half
  // while the matrix cores run step kt-1's second half from registers, so the
  // barrier never leaves the matrix cores without operands.
  const int nk = K / 64;
  SPA_ISSUE24(0, 0);
  if (nk > 1) SPA_ISSUE24(1, 1);
  SPA_WAIT24(nk > 1);
  bare_barrier();
  if (nk > 2) SPA_ISSUE24(2, 2);
  SPA_READ24(0, 0);
  SPA_READ24(0, 1);
  SPA_MMA24(0);
  int st = 0;
  for (int kt = 1; kt < nk; ++kt) {
    st = st == 2 ? 0 : st + 1;                 // kt % 3
    SPA_WAIT24(kt + 1 < nk);                   // step kt landed (kt+1 may be in flight)
    bare_barrier();                            // B_kt
    if (kt + 2 < nk) SPA_ISSUE24(kt + 2, st == 0 ? 2 : st - 1);
    SPA_READ24(st, 0);
    SPA_MMA24(1);                              // step kt-1, second half
    SPA_READ24(st, 1);
    SPA_MMA24(0);                              // step kt, first half
  }
  SPA_MMA24(1);                                // last step, second half
#undef SPA_ISSUE24
#undef SPA_WAIT24
#undef SPA_READ24
#undef SPA_MMA24

  ts.park(s_nu, s_eta, s_rs);
  __syncthreads();                             // every wave is done with the ring
  // the wave's output block: the weight ring (3 x 32 KB) first, then the activation ring
  constexpr int BLK = WM * WN * 2;
  static_assert(3 * BST % BLK == 0 && NW * BLK <= 3 * BST + 3 * AST, "output blocks fit the ring");
  const int off = wv * BLK;
  uint16_t* blk = reinterpret_cast<uint16_t*>(off < 3 * BST ? sB + off : sA + (off - 3 * BST));
  store_tile_lds<DT, FM, FN>(p, acc, m0, n0, wm0, wn0, g, l32, lane, s_nu, s_eta, s_rs, blk);
}

// ---------------------------------------------------------------------------
// Dense MFMA on masked rows (n:m other than 2:4): BM = 256 tokens x BN = 128
// outputs per workgroup, waves in a 4 x 2 grid of 64 x 64 (2 x 2 fragments of
// 32 x 32).  A stage is 256 activation rows + 128 weight rows of 128 B; each
// wave issues six 1 KB direct loads per step, so vmcnt <= 6 means "the older
// step in flight has landed".  Rows past t (or n_out) re-read the last row;
// their outputs are never stored.  Chunk c of any row r sits at c ^ ((r>>1)&7).
//
// EPI = 1 is the up-projection of a squared-ReLU FFN whose activation feeds a
// 2:4 layer ("Accelerating Transformer training and inference with 2:4
// sparsity and Squared-ReLU" s3.1: one kernel applies the activation, prunes
// and packs): the tile's outputs u are rounded to the storage dtype, squared
// after max(u, 0) and rounded again (what a separate pass would store), held
// in the freed LDS ring as two 64-channel steps, then pruned 2:4 by magnitude
// and packed into the tiled operand of the 2:4 GEMM -- the activation never
// reaches HBM dense.
// ---------------------------------------------------------------------------
template <int DT, int EPI>
__global__ void __launch_bounds__(512, 1) k_gemm_dense(PrefillArgs p) {
  constexpr int BM = 256, BN = 128;
  constexpr int WM = 64, WN = 64, FM = 2, FN = 2;
  using V8 = typename Frag<DT>::V8;
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[BM * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[BM * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sA2[BM * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[BN * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[BN * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sB2[BN * 64];
  __shared__ float s_nu[BM], s_eta[BM], s_rs[BN];

  const int T = p.t, K = p.k, N = p.n_out;
  int tm, tn;
  xcd_tile(T, N, BM, BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  TileScalars<BM, BN> ts;
  ts.fetch(p, m0, n0);

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int wm0 = (wv >> 1) * WM, wn0 = (wv & 1) * WN;

  const char* baseA = static_cast<const char*>(p.a_vals) + (size_t)m0 * K * 2;
  const char* baseW = static_cast<const char*>(p.w) + (size_t)n0 * K * 2;
  uint32_t offA[4], offB[2];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int r = 32 * wv + 8 * h + (lane >> 3);
    const int rr = min(m0 + r, T - 1) - m0;
    offA[h] = (uint32_t)rr * (uint32_t)K * 2u + (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) * 16);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 16 * wv + 8 * h + (lane >> 3);
    const int rr = min(n0 + r, N - 1) - n0;
    offB[h] = (uint32_t)rr * (uint32_t)K * 2u + (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) * 16);
  }
  const int q = (l32 >> 1) & 7;
  int ldsA[4], ldsB[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    ldsA[s] = (wm0 + l32) * 128 + (((2 * s + g) ^ q) * 16);
    ldsB[s] = (wn0 + l32) * 128 + (((2 * s + g) ^ q) * 16);
  }

#define SPA_ISSUED(KT, SA, SB)                                                     \
  do {                                                                             \
    const char* a_ = baseA + (size_t)(KT) * 128;                                   \
    const char* w_ = baseW + (size_t)(KT) * 128;                                   \
    const uint32_t la_ = lds_addr(SA) + wv * 4096, lb_ = lds_addr(SB) + wv * 2048; \
    lds_dma16(a_, offA[0], la_);                                                   \
    lds_dma16(a_, offA[1], la_ + 1024);                                            \
    lds_dma16(a_, offA[2], la_ + 2048);                                            \
    lds_dma16(a_, offA[3], la_ + 3072);                                            \
    lds_dma16(w_, offB[0], lb_);                                                   \
    lds_dma16(w_, offB[1], lb_ + 1024);                                            \
  } while (0)

#define SPA_COMPUTED(SA, SB)                                                                         \
  do {                                                                                              \
    const char* a_ = reinterpret_cast<const char*>(SA);                                             \
    const char* b_ = reinterpret_cast<const char*>(SB);                                             \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                                 \
      V8 bf[FN];                                                                                    \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                                \
        bf[j] = as_vec<V8>(*reinterpret_cast<const uint4*>(b_ + ldsB[s] + j * 4096));              \
      _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                              \
        const V8 af = as_vec<V8>(*reinterpret_cast<const uint4*>(a_ + ldsA[s] + i * 4096));         \
        _Pragma("unroll") for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<DT>(af, bf[j], acc[i][j]); \
      }                                                                                             \
    }                                                                                               \
  } while (0)

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / 64;
  const int nq = nk / 3, nr = nk - 3 * nq;
  SPA_ISSUED(0, sA0, sB0);
  if (nk > 1) SPA_ISSUED(1, sA1, sB1);
  for (int qq = 0; qq < nq; ++qq) {
    const int kt = 3 * qq;
    wait_vm<6>(kt + 1 < nk);
    bare_barrier();
    SPA_ISSUED(kt + 2, sA2, sB2);
    SPA_COMPUTED(sA0, sB0);
    wait_vm<6>(1);
    bare_barrier();
    if (kt + 3 < nk) SPA_ISSUED(kt + 3, sA0, sB0);
    SPA_COMPUTED(sA1, sB1);
    wait_vm<6>(kt + 3 < nk);
    bare_barrier();
    if (kt + 4 < nk) SPA_ISSUED(kt + 4, sA1, sB1);
    SPA_COMPUTED(sA2, sB2);
  }
  if (nr >= 1) {
    wait_vm<6>(nr == 2);
    bare_barrier();
    SPA_COMPUTED(sA0, sB0);
  }
  if (nr == 2) {
    wait_vm<6>(0);
    bare_barrier();
    SPA_COMPUTED(sA1, sB1);
  }
#undef SPA_ISSUED
#undef SPA_COMPUTED

  if constexpr (EPI == 0) {
    ts.park(s_nu, s_eta, s_rs);
    __syncthreads();                           // every wave is done with the ring
    // the wave's 8 KB output block: waves 0-3 in the first activation stage, 4-7 in the second
    static_assert(WM * WN * 4 <= BM * 64, "four output blocks per activation stage");
    uint16_t* blk = (wv < 4 ? sA0 : sA1) + (wv & 3) * (WM * WN);
    store_tile_lds<DT, FM, FN>(p, acc, m0, n0, wm0, wn0, g, l32, lane, s_nu, s_eta, s_rs, blk);
  } else {
    // every wave is past its last read of the ring: step 0 of the tile (its
    // columns 0..63) goes to sA0, step 1 to sA1, row-major [256][64]
    __syncthreads();
    uint16_t* s_step = (wn0 == 0) ? sA0 : sA1;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tr = wm0 + 32 * i + 8 * (r / 4) + 4 * g + (r % 4);
          const int tc = 32 * j + l32;                          // column inside the step
          const float u = to_f32<DT>(from_f32<DT>(acc[i][j][r]));
          s_step[tr * 64 + tc] = from_f32<DT>(relu2<DT>(u));
        }
    __syncthreads();
    // 2 steps x 256 rows x 4 segments of 16 channels (four 2:4 blocks each)
    const int step0 = n0 / 64;
    for (int e = threadIdx.x; e < 2 * BM * 4; e += 512) {
      const int s = e >> 10, rr = (e >> 2) & (BM - 1), q = e & 3;
      const int row = m0 + rr;
      if (row >= T || n0 + 64 * s >= N) continue;
      const uint16_t* src = (s ? sA1 : sA0) + rr * 64 + 16 * q;
      const uint4 lo4 = *reinterpret_cast<const uint4*>(src);
      const uint4 hi4 = *reinterpret_cast<const uint4*>(src + 8);
      const uint32_t w8[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
      uint32_t wds[4], meta = 0;
      uint32_t pos[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint32_t bits[4];
        float sc[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint32_t wv2 = w8[(4 * b + jj) >> 1];
          bits[jj] = ((4 * b + jj) & 1) ? (wv2 >> 16) : (wv2 & 0xFFFFu);
          sc[jj] = __builtin_fabsf(to_f32<DT>((uint16_t)bits[jj]));
        }
        // rank rule: j < q beats q unless q's score is strictly larger
        int rank[4] = {0, 0, 0, 0};
#pragma unroll
        for (int j0 = 0; j0 < 4; ++j0)
#pragma unroll
          for (int j1 = j0 + 1; j1 < 4; ++j1) {
            const bool w0 = sc[j0] >= sc[j1];
            rank[j1] += w0 ? 1 : 0;
            rank[j0] += w0 ? 0 : 1;
          }
        uint32_t kb = 0;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) kb |= (rank[jj] < 2 ? 1u : 0u) << jj;
        const uint32_t lo = __builtin_ctz(kb), hi = 31 - __builtin_clz(kb);
        meta |= (lo | (hi << 2)) << (4 * b);
        uint32_t vlo = bits[0], vhi = bits[0];
#pragma unroll
        for (int jj = 1; jj < 4; ++jj) {
          vlo = (int)lo == jj ? bits[jj] : vlo;
          vhi = (int)hi == jj ? bits[jj] : vhi;
        }
        wds[b] = vlo | (vhi << 16);
        pos[b] = lo | (hi << 8);
      }
      const size_t rowpos = (size_t)(step0 + s) * p.out_t_pad + row;
      reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out_vals) + rowpos * 32)[q] =
          make_uint4(wds[0], wds[1], wds[2], wds[3]);
      p.out_meta[rowpos * 4 + q] = (uint16_t)meta;
      if (p.out_idx) {
        // positions of the segment's four blocks, two bytes each, row-major [t][n_out/2]
        uint8_t* ip = p.out_idx + (size_t)row * (N / 2) + (size_t)(n0 + 64 * s + 16 * q) / 2;
        *reinterpret_cast<uint2*>(ip) = make_uint2(pos[0] | (pos[1] << 16), pos[2] | (pos[3] << 16));
      }
    }
  }
}

// The CUs of the current device (queried once).
static int device_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 256;
    return n > 0 ? n : 256;
  }();
  return cus;
}

// One workgroup per CU at a time.  When the 256 x 256 tiles leave a last
// round at most three quarters full, whole rounds of them cover the first
// columns and one round of 256 x 192 tiles the rest: 2048 x 4096 -> 14336
// runs 256 + 256 workgroups (about 1.75 tile times) instead of 448 (two).
// Returns where the 192-column tiles start (n_out: no split).
static int balanced_cols(int t, int n_out) {
  const int tm = (t + 255) / 256, tn = (n_out + 255) / 256, cus = device_cus();
  const int full = tm * tn / cus, rem = tm * tn - full * cus;
  if (full >= 1 && rem > 0 && 4 * rem <= 3 * cus && (full * cus) % tm == 0) {
    const int c1 = full * cus / tm * 256;
    if (c1 < n_out && tm * ((n_out - c1 + 191) / 192) <= cus) return c1;
  }
  return n_out;
}

template <int DT>
static void gemm24_launch(const PrefillArgs& a, hipStream_t st) {
  // Up to 128 k steps per tile the 256-column tiles use 16 waves (four per
  // SIMD), beyond that 8: level with each other where both were measured.
  const bool w16 = a.k <= 8192;
  const int tm = (a.t + 255) / 256, n1 = balanced_cols(a.t, a.n_out);
  PrefillArgs b = a;
  b.col0 = 0;
  b.col1 = n1;
  const int tiles = tm * ((n1 + 255) / 256);
  if (w16) hipLaunchKernelGGL((k_gemm24<DT, 16>), dim3(tiles), dim3(1024), 0, st, b);
  else hipLaunchKernelGGL((k_gemm24<DT, 8>), dim3(tiles), dim3(512), 0, st, b);
  if (n1 < a.n_out) {
    b.col0 = n1;
    b.col1 = a.n_out;
    hipLaunchKernelGGL((k_gemm24<DT, 12>), dim3(tm * ((a.n_out - n1 + 191) / 192)), dim3(768), 0, st, b);
  }
}

hipError_t launch_gemm(int dtype, const PrefillArgs& a, hipStream_t st) {
  if (a.t == 0) return hipSuccess;
  if (a.sparse24) {
    if (dtype == SPA_F16) gemm24_launch<SPA_F16>(a, st);
    else gemm24_launch<SPA_BF16>(a, st);
  } else {
    const int tiles = ((a.t + 255) / 256) * ((a.n_out + 127) / 128);
    if (dtype == SPA_F16) hipLaunchKernelGGL((k_gemm_dense<SPA_F16, 0>), dim3(tiles), dim3(512), 0, st, a);
    else hipLaunchKernelGGL((k_gemm_dense<SPA_BF16, 0>), dim3(tiles), dim3(512), 0, st, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// FP8 2:4 GEMM ("Accelerating Transformer training and inference with 2:4
// sparsity and Squared-ReLU" s2.1, s3.1: the sparse GEMM on FP8 with row
// scales).  gfx950's v_smfmac_f32_32x32x64_fp8_fp8 takes a whole 64-channel
// step per instruction: A lane l holds row l % 32's 16 kept e4m3 codes of
// logical channels [32g, 32g + 32) (g = l / 32) with two position bits each
// in one 32-bit word; B lane l holds column l % 32's codes of channels
// 16g .. 16g + 15 and 32 + 16g .. 32 + 16g + 15; D as for the 16-bit
// instruction.  Same 256 x 256 tile and three-stage ring of direct loads as
// k_gemm24, at half the bytes: per step and row 32 B of codes + 8 B of
// positions (activations) and 64 B of codes (weights).  16 waves of 64 x 64
// outputs (four waves per SIMD; 8 waves of 128 x 64 ran 5 % slower).  Per
// stage every wave loads one 1 KB run of weight codes (16 rows); waves 0-7
// also load one run of activation codes (32 rows) and one of positions (32
// rows).  All of a step's fragment reads are issued before its products.
// The 16-byte chunks are XOR-swizzled against bank conflicts: chunk c of
// activation row r sits at c ^ ((r >> 3) & 1), of weight row r at
// c ^ ((r >> 2) & 3).  y = nu_i * sx_i * sw_j * acc + eta_i * s_j.
// ---------------------------------------------------------------------------
template <int DT, int NW>
__global__ void __launch_bounds__(NW * 64, 1) k_gemm24_fp8(PrefillArgs p) {
  static_assert(NW == 12 || NW == 16, "waves of 64 x 64 over 192 or 256 columns");
  constexpr int BM = 256, BN = NW == 12 ? 192 : 256;
  constexpr int WM = 64, WN = 64, FM = 2, FN = 2, WC = BN / WN;
  constexpr int AST = BM * 40, BST = BN * 64;               // bytes per stage
  typedef int v4i __attribute__((ext_vector_type(4)));
  typedef int v8i __attribute__((ext_vector_type(8)));
  // one ring: three activation stages, then three weight stages, sized up
  // so that it also holds the waves' 8 KB output blocks
  constexpr int RING = 3 * (AST + BST) > NW * 8192 ? 3 * (AST + BST) : NW * 8192;
  static_assert((3 * AST) % 1024 == 0, "weight stages 1 KB aligned");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[RING];
  unsigned char* const sA = ring;
  unsigned char* const sB = ring + 3 * AST;
  __shared__ float s_nu[BM], s_eta[BM], s_rs[BN], s_sx[BM], s_sw[BN];

  const int K = p.k, N = p.n_out, TP = p.t_pad;
  int tm, tn;
  xcd_tile(p.t, p.col1 - p.col0, BM, BN, tm, tn);
  const int m0 = tm * BM, n0 = p.col0 + tn * BN;
  TileScalars<BM, BN> ts;
  ts.fetch(p, m0, n0);
  const float sx_own = (int)threadIdx.x < BM ? p.sx[min(m0 + (int)threadIdx.x, p.t - 1)] : 0.f;
  const float sw_own = (int)threadIdx.x < BN ? p.sw[min(n0 + (int)threadIdx.x, N - 1)] : 0.f;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int wm0 = (wv / WC) * WM, wn0 = (wv % WC) * WN;
  const bool loads_a = wv < 8;                              // wave-uniform

  const char* baseA = static_cast<const char*>(p.a_vals) + (size_t)m0 * 32;
  const char* baseM = reinterpret_cast<const char*>(p.a_meta) + (size_t)m0 * 8;
  const char* baseW = static_cast<const char*>(p.w) + (size_t)n0 * K;
  const size_t stepA = (size_t)TP * 32, stepM = (size_t)TP * 8;
  const int wa = wv & 7;
  const int ra = 32 * wa + (lane >> 1);
  const uint32_t offA = (uint32_t)(ra * 32 + (((lane & 1) ^ ((ra >> 3) & 1)) * 16));
  const uint32_t offM = (uint32_t)((wa * 64 + lane) * 4);
  const int rb = 16 * wv + (lane >> 2);
  const int rbc = min(n0 + rb, N - 1) - n0;
  const uint32_t offB = (uint32_t)rbc * (uint32_t)K + (uint32_t)(((lane & 3) ^ ((rb >> 2) & 3)) * 16);
  const uint32_t ldsA0 = lds_addr(sA), ldsB0 = lds_addr(sB);

#define SPA_ISSUE8W(KT, ST)                                                                  \
  do {                                                                                       \
    lds_dma16(baseW + (size_t)(KT) * 64, offB, ldsB0 + (ST) * BST + wv * 1024);              \
    if (loads_a) {                                                                           \
      lds_dma16(baseA + (size_t)(KT) * stepA, offA, ldsA0 + (ST) * AST + wa * 1024);         \
      lds_dma4(baseM + (size_t)(KT) * stepM, offM, ldsA0 + (ST) * AST + BM * 32 + wa * 256); \
    }                                                                                        \
  } while (0)

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / 64;
  SPA_ISSUE8W(0, 0);
  if (nk > 1) SPA_ISSUE8W(1, 1);
  int st = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // step kt landed (kt+1 may be in flight: 3 loads for waves 0-7, 1 for the others)
    if (loads_a) wait_vm<3>(kt + 1 < nk);
    else wait_vm<1>(kt + 1 < nk);
    bare_barrier();                              // every wave's copies visible; stage (kt+2)%3 free
    if (kt + 2 < nk) SPA_ISSUE8W(kt + 2, st == 0 ? 2 : st - 1);
    const unsigned char* a_ = sA + st * AST;
    const unsigned char* b_ = sB + st * BST;
    v8i bf[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wn0 + 32 * j + l32;
      const int q = (row >> 2) & 3;
      const uint4 lo = *reinterpret_cast<const uint4*>(b_ + row * 64 + ((g ^ q) * 16));
      const uint4 hi = *reinterpret_cast<const uint4*>(b_ + row * 64 + (((2 + g) ^ q) * 16));
      bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    v4i af[FM];
    int ix[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm0 + 32 * i + l32;
      const uint4 av = *reinterpret_cast<const uint4*>(a_ + row * 32 + ((g ^ ((row >> 3) & 1)) * 16));
      ix[i] = *reinterpret_cast<const int*>(a_ + BM * 32 + row * 8 + g * 4);
      af[i] = v4i{(int)av.x, (int)av.y, (int)av.z, (int)av.w};
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(af[i], bf[j], acc[i][j], ix[i], 0, 0);
    st = st == 2 ? 0 : st + 1;
  }
#undef SPA_ISSUE8W

  ts.park(s_nu, s_eta, s_rs);
  if ((int)threadIdx.x < BM) s_sx[threadIdx.x] = sx_own * ts.nu;   // nu_i * sx_i
  if ((int)threadIdx.x < BN) s_sw[threadIdx.x] = sw_own;
  __syncthreads();                             // every wave is done with the ring
  static_assert(NW * WM * WN * 2 <= RING, "output blocks fit the ring");
  uint16_t* blk = reinterpret_cast<uint16_t*>(ring + wv * (WM * WN * 2));
  store_tile_lds<DT, FM, FN, true>(p, acc, m0, n0, wm0, wn0, g, l32, lane, s_sx, s_eta, s_rs, blk, s_sw);
}

template <int DT>
static void gemm24_fp8_launch(const PrefillArgs& a, hipStream_t st) {
  // the column split of gemm24_launch: whole rounds of 256-column tiles, then
  // one round of 192-column tiles
  const int tm = (a.t + 255) / 256, n1 = balanced_cols(a.t, a.n_out);
  PrefillArgs b = a;
  b.col0 = 0;
  b.col1 = n1;
  hipLaunchKernelGGL((k_gemm24_fp8<DT, 16>), dim3(tm * ((n1 + 255) / 256)), dim3(1024), 0, st, b);
  if (n1 < a.n_out) {
    b.col0 = n1;
    b.col1 = a.n_out;
    hipLaunchKernelGGL((k_gemm24_fp8<DT, 12>), dim3(tm * ((a.n_out - n1 + 191) / 192)), dim3(768), 0, st, b);
  }
}

hipError_t launch_gemm_fp8(int dtype, const PrefillArgs& a, hipStream_t st) {
  if (a.t == 0) return hipSuccess;
  if (dtype == SPA_F16) gemm24_fp8_launch<SPA_F16>(a, st);
  else gemm24_fp8_launch<SPA_BF16>(a, st);
  return hipGetLastError();
}

// Weight rows to e4m3 codes with one scale per row (max |w| / 448); one
// workgroup per row, k % 8 == 0.
template <int DT>
__global__ void __launch_bounds__(256) k_quant_rows(const uint16_t* __restrict__ w, int k, uint8_t* __restrict__ codes,
                                                    float* __restrict__ scale) {
  __shared__ float s_mx[4];
  const uint16_t* row = w + (size_t)blockIdx.x * k;
  float mx = 0.f;
  for (int q = threadIdx.x; q < k / 8; q += 256) {
    const uint4 u = reinterpret_cast<const uint4*>(row)[q];
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, __builtin_fabsf(elem16<DT>(u, e)));
  }
  const float amax = block_max(mx, s_mx);
  float sc, inv;
  fp8_scales(amax, sc, inv);
  if (threadIdx.x == 0) scale[blockIdx.x] = sc;
  uint8_t* out = codes + (size_t)blockIdx.x * k;
  for (int q = threadIdx.x; q < k / 8; q += 256) {
    const uint4 u = reinterpret_cast<const uint4*>(row)[q];
    const uint32_t lo = fp8_pair(elem16<DT>(u, 0) * inv, elem16<DT>(u, 1) * inv) |
                        (fp8_pair(elem16<DT>(u, 2) * inv, elem16<DT>(u, 3) * inv) << 16);
    const uint32_t hi = fp8_pair(elem16<DT>(u, 4) * inv, elem16<DT>(u, 5) * inv) |
                        (fp8_pair(elem16<DT>(u, 6) * inv, elem16<DT>(u, 7) * inv) << 16);
    reinterpret_cast<uint2*>(out)[q] = make_uint2(lo, hi);
  }
}

hipError_t launch_quant_rows(int dtype, const void* w, int n_out, int k, uint8_t* codes, float* scale,
                             hipStream_t st) {
  if (n_out == 0) return hipSuccess;
  if (dtype == SPA_F16)
    hipLaunchKernelGGL(k_quant_rows<SPA_F16>, dim3(n_out), dim3(256), 0, st, static_cast<const uint16_t*>(w), k, codes,
                       scale);
  else
    hipLaunchKernelGGL(k_quant_rows<SPA_BF16>, dim3(n_out), dim3(256), 0, st, static_cast<const uint16_t*>(w), k,
                       codes, scale);
  return hipGetLastError();
}

hipError_t launch_ffn_up(int dtype, const PrefillArgs& a, hipStream_t st) {
  if (a.t == 0) return hipSuccess;
  const int tiles = ((a.t + 255) / 256) * ((a.n_out + 127) / 128);
  if (dtype == SPA_F16) hipLaunchKernelGGL((k_gemm_dense<SPA_F16, 1>), dim3(tiles), dim3(512), 0, st, a);
  else hipLaunchKernelGGL((k_gemm_dense<SPA_BF16, 1>), dim3(tiles), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace spa

// Decode: pruned activations times a channel-major weight, 1..32 tokens.
//
// The weight is stored channel-major (wt[k][n_out]), so a channel that no
// token of the call keeps is a whole row of wt that is never read: the
// HBM bytes fall by about n/m (guide s1.1: zero activations need not be
// moved; s12.3: bandwidth first).  The shifted form
//   y = nu * (x_hat * mask) W^T + eta * (W 1)
// (guide s3.1 with the rescale of s3.2) reads only kept rows; W 1 is the
// precomputed row sum.
//
// Work split: workgroup (tile, split) owns columns [tile*C, tile*C + C) and
// channels [split*k_len, (split+1)*k_len).  Each writes a float32 partial
// row; the last workgroup of a tile to finish (ticket counter) adds the
// partials in split order, so results do not depend on arrival order, and
// applies the epilogue.  Counters are left at zero for the next call.
//
// Two variants:
//  * fused (t <= 4): each workgroup prunes its own channel range in LDS
//    (the same few thousand comparisons in every tile) and streams the kept
//    rows with float32 VALU FMAs, 16 bytes per lane per row;
//  * mask + stream (t > 4, 16-bit): one mask kernel prunes every channel
//    once, recording which tokens keep each channel and the kept values;
//    the stream kernel reads the union of kept rows once and runs the
//    tokens x rows x columns product on matrix cores (mfma 16x16x32).
#include "spa_common.h"
#include "spa_launch.h"

namespace spa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTok = 32;

// ---------------------------------------------------------------------------
// Epilogue shared by both variants: arrive at the tile's ticket; the last
// arrival reduces the partials and writes y.
// ---------------------------------------------------------------------------
template <int DT>
__device__ void finish_tile(const DecodeArgs& a, int tile, int split, const float* s_eta, int* s_flag,
                            float* s_nu) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned ticket = atomicAdd(&a.counters[tile], 1u);
    *s_flag = (ticket == (unsigned)(a.splits - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!*s_flag) return;
  __threadfence();

  const int T = a.t;
  if ((int)threadIdx.x < T) {
    float nu = 1.f;
    if (a.var) {
      const int i = threadIdx.x;
      double s[4] = {0.0, 0.0, 0.0, 0.0};
      // the statistics of every channel group, in group order
      const int groups = a.mask_groups > 0 ? a.mask_groups : a.splits;
      const double* base = a.mask_groups > 0 ? a.stats : a.stats + (size_t)tile * a.splits * T * 4;
      // fused path: every tile keeps its own copy, so the reducer never waits on another tile
      for (int g = 0; g < groups; ++g)
        for (int q = 0; q < 4; ++q) s[q] += base[((size_t)g * T + i) * 4 + q];
      const double kk = (double)a.k;
      const double vf = s[1] / kk - (s[0] / kk) * (s[0] / kk);
      const double vm = s[3] / kk - (s[2] / kk) * (s[2] / kk);
      if (vm > 0.0) nu = (float)__builtin_sqrt(vf / vm);
    }
    s_nu[threadIdx.x] = nu;
    if (tile == 0 && a.nu_out) a.nu_out[threadIdx.x] = nu;
  }
  __syncthreads();

  using T_ = typename Dt<DT>::T;
  T_* y = static_cast<T_*>(a.y);
  const int c0 = tile * a.col_tile;
  const int cw = min(a.col_tile, a.n_out - c0);
  for (int p = threadIdx.x; p < T * cw; p += 256) {
    const int i = p / cw, cc = p % cw, col = c0 + cc;
    float acc = 0.f;
    for (int s = 0; s < a.splits; ++s) acc += a.partial[((size_t)s * T + i) * a.n_out + col];
    float v = s_nu[i] * acc;
    if (a.shift != SPA_SHIFT_NONE) v += s_eta[i] * a.row_sum[col];
    y[(size_t)i * a.n_out + col] = from_f32<DT>(v);
  }
  if (threadIdx.x == 0) a.counters[tile] = 0u;
}

// ---------------------------------------------------------------------------
// Fused variant (t <= TOK <= 8).
// ---------------------------------------------------------------------------
template <int DT, int M, int TOK>
__global__ void __launch_bounds__(256) k_decode_fused(DecodeArgs a) {
  using T = typename Dt<DT>::T;
  constexpr int CPL = 16 / Dt<DT>::bytes;   // columns per lane (one 16-byte load)
  constexpr int C = 64 * CPL;               // column tile
  constexpr int UNR = 8;                    // rows in flight per lane

  extern __shared__ unsigned char s_dyn[];
  __shared__ double s_red[4];
  __shared__ int s_cnt[4];
  __shared__ float s_eta[TOK];
  __shared__ float s_nu[TOK];
  __shared__ int s_flag;

  const int T_ = a.t;
  const int tile = blockIdx.x % a.tiles;
  const int split = blockIdx.x / a.tiles;
  const int kb = split * a.k_len;
  const int KL = min(a.k_len, a.k - kb);    // the last split may be shorter
  const T* x = static_cast<const T*>(a.x);

  // LDS carve-up (strides use KL; sizes were reserved for k_len)
  float* s_sc = reinterpret_cast<float*>(s_dyn);                // [TOK][KL] scores
  float* s_coef = s_sc + TOK * a.k_len;                         // [TOK][KL] x_hat, then kept-or-0
  int* s_rows = reinterpret_cast<int*>(s_coef + TOK * a.k_len); // [KL] token masks, then union rows
  uint8_t* s_keep = reinterpret_cast<uint8_t*>(s_rows + a.k_len);  // [TOK][KL]
  float* s_acc = reinterpret_cast<float*>(s_keep + ((TOK * a.k_len + 15) & ~15));  // [4][TOK][C]

  // 1. shift
  for (int i = 0; i < T_; ++i) {
    float e = 0.f;
    if (a.shift == SPA_SHIFT_TOKEN_MEAN && a.eta == nullptr) {
      double s = 0.0;
      for (int c = threadIdx.x; c < a.k; c += 256) s += (double)to_f32<DT>(x[(size_t)i * a.k + c]);
      e = (float)(block_sum(s, s_red) / (double)a.k);
    } else if (a.eta != nullptr) {
      e = a.eta[i];
    }
    if (threadIdx.x == 0) s_eta[i] = e;
  }
  __syncthreads();

  // 2. channel factor and scores
  for (int c = threadIdx.x; c < KL; c += 256) {
    float f = 1.f;
    if (a.score == SPA_SCORE_WEIGHT) {
      f = a.chan_scale[kb + c];
    } else if (a.score == SPA_SCORE_CLACT) {
      float acc = 0.f;
      for (int p = 0; p < T_; ++p) acc = clact_accumulate(acc, to_f32<DT>(x[(size_t)p * a.k + kb + c]) - s_eta[p]);
      f = sqrt_rn(acc);
    }
    for (int i = 0; i < T_; ++i) {
      const float xh = to_f32<DT>(x[(size_t)i * a.k + kb + c]) - s_eta[i];
      s_coef[i * KL + c] = xh;
      s_sc[i * KL + c] = a.score == SPA_SCORE_MAGNITUDE ? __builtin_fabsf(xh) : __builtin_fabsf(xh) * f;
    }
  }
  __syncthreads();

  // 3. per-element rank within its block
  for (int c = threadIdx.x; c < KL; c += 256) {
    const int j = c % M, base = c - j;
    uint32_t tokmask = 0;
    for (int i = 0; i < T_; ++i) {
      const float* sc = s_sc + i * KL + base;
      const float me = sc[j];
      int rank = 0;
#pragma unroll
      for (int q = 0; q < M; ++q) rank += beats(sc[q], q, me, j) ? 1 : 0;
      const bool keep = rank < a.n;
      s_keep[i * KL + c] = keep ? 1 : 0;
      if (keep) tokmask |= 1u << i;
    }
    s_rows[c] = (int)tokmask;
  }
  __syncthreads();

  // 3b. in-block positions (one workgroup per split writes them), kept-or-zero
  //     coefficients, variance statistics of this channel range
  const bool write_idx = (a.idx_out != nullptr) && tile == 0;
  for (int c = threadIdx.x; c < KL; c += 256) {
    const int j = c % M, base = c - j;
    for (int i = 0; i < T_; ++i) {
      if (s_keep[i * KL + c]) {
        if (write_idx) {
          int before = 0;
          for (int q = 0; q < j; ++q) before += s_keep[i * KL + base + q];
          a.idx_out[(size_t)i * (a.k / M * a.n) + (size_t)(kb + base) / M * a.n + before] = (uint8_t)j;
        }
      }
    }
  }
  if (a.var) {
    for (int i = 0; i < T_; ++i) {
      double ts[4] = {0.0, 0.0, 0.0, 0.0};
      for (int c = threadIdx.x; c < KL; c += 256) {
        const double v = (double)s_coef[i * KL + c];
        ts[0] += v; ts[1] += v * v;
        if (s_keep[i * KL + c]) { ts[2] += v; ts[3] += v * v; }
      }
      for (int q = 0; q < 4; ++q) {
        const double tot = block_sum(ts[q], s_red);
        if (threadIdx.x == 0) a.stats[(((size_t)tile * a.splits + split) * T_ + i) * 4 + q] = tot;
      }
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < KL; c += 256)
    for (int i = 0; i < T_; ++i)
      if (!s_keep[i * KL + c]) s_coef[i * KL + c] = 0.f;

  // 4. union of kept rows, ascending
  int U = 0;
  for (int c0 = 0; c0 < KL; c0 += 256) {
    const int c = c0 + threadIdx.x;
    const bool f = c < KL && s_rows[c] != 0;
    int total;
    const int pos = block_exclusive_count(f, s_cnt, &total);
    if (f) s_acc[U + pos] = __int_as_float(c);  // s_acc is free until the main loop ends
    U += total;
  }
  __syncthreads();
  for (int u = threadIdx.x; u < U; u += 256) s_rows[u] = __float_as_int(s_acc[u]);
  __syncthreads();

  // 5. stream the kept rows of wt
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int col = tile * C + lane * CPL;
  const bool cvalid = col < a.n_out;
  float acc[TOK][CPL];
#pragma unroll
  for (int i = 0; i < TOK; ++i)
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[i][e] = 0.f;

  const T* wt = static_cast<const T*>(a.wt);
  for (int u0 = wv; u0 < U; u0 += 4 * UNR) {
    uint4 wv16[UNR];
    int rr[UNR];
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      const int u = u0 + 4 * r;
      rr[r] = u < U ? s_rows[u] : -1;
      if (rr[r] >= 0 && cvalid)
        wv16[r] = *reinterpret_cast<const uint4*>(wt + (size_t)(kb + rr[r]) * a.n_out + col);
      else
        wv16[r] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      if (rr[r] < 0) continue;
      float wf[CPL];
      if constexpr (DT == SPA_F32) {
        wf[0] = __uint_as_float(wv16[r].x); wf[1] = __uint_as_float(wv16[r].y);
        wf[2] = __uint_as_float(wv16[r].z); wf[3] = __uint_as_float(wv16[r].w);
      } else {
#pragma unroll
        for (int e = 0; e < CPL; ++e) wf[e] = elem16<DT>(wv16[r], e);
      }
#pragma unroll
      for (int i = 0; i < TOK; ++i) {
        if (i < T_) {
          const float cf = s_coef[i * KL + rr[r]];
#pragma unroll
          for (int e = 0; e < CPL; ++e) acc[i][e] += cf * wf[e];
        }
      }
    }
  }
  __syncthreads();  // s_acc held the union list

  // 6. reduce the four waves, write this split's partial
#pragma unroll
  for (int i = 0; i < TOK; ++i)
#pragma unroll
    for (int e = 0; e < CPL; ++e) s_acc[(wv * TOK + i) * C + lane * CPL + e] = acc[i][e];
  __syncthreads();
  const int c0 = tile * C;
  const int cw = min(C, a.n_out - c0);
  for (int p = threadIdx.x; p < T_ * cw; p += 256) {
    const int i = p / cw, cc = p % cw;
    const float v = ((s_acc[(0 * TOK + i) * C + cc] + s_acc[(1 * TOK + i) * C + cc]) + s_acc[(2 * TOK + i) * C + cc]) +
                    s_acc[(3 * TOK + i) * C + cc];
    a.partial[((size_t)split * T_ + i) * a.n_out + c0 + cc] = v;
  }
  finish_tile<DT>(a, tile, split, s_eta, &s_flag, s_nu);
}

// ---------------------------------------------------------------------------
// Mask kernel (t > 4): 64 channels x all tokens per workgroup.
// tokmask[c]: bit i set when token i keeps channel c.  coef[c][i]: kept
// x_hat rounded to the storage dtype (0 when pruned), tokens padded to 32.
// ---------------------------------------------------------------------------
template <int DT, int M>
__global__ void __launch_bounds__(256) k_decode_mask(DecodeArgs a) {
  using T = typename Dt<DT>::T;
  constexpr int KM = 64;
  __shared__ float s_sc[kMaxTok][KM];
  __shared__ float s_xh[kMaxTok][KM];
  __shared__ uint8_t s_keep[kMaxTok][KM];
  __shared__ uint32_t s_tm[KM];
  __shared__ float s_f[KM];
  __shared__ double s_red[4];
  const int T_ = a.t;
  const int kb = blockIdx.x * KM;
  const int KV = min(KM, a.k - kb);          // a whole number of m-blocks
  const T* x = static_cast<const T*>(a.x);
  const float* eta = a.eta;

  if ((int)threadIdx.x < KM) {
    const int c = threadIdx.x;
    s_tm[c] = 0u;
    float f = 1.f;
    if (c < KV) {
      if (a.score == SPA_SCORE_WEIGHT) {
        f = a.chan_scale[kb + c];
      } else if (a.score == SPA_SCORE_CLACT) {
        float acc = 0.f;
        for (int p = 0; p < T_; ++p)
          acc = clact_accumulate(acc, to_f32<DT>(x[(size_t)p * a.k + kb + c]) - (eta ? eta[p] : 0.f));
        f = sqrt_rn(acc);
      }
    }
    s_f[c] = f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < T_ * KM; e += 256) {
    const int i = e / KM, c = e % KM;
    float xh = 0.f;
    if (c < KV) xh = to_f32<DT>(x[(size_t)i * a.k + kb + c]) - (eta ? eta[i] : 0.f);
    s_xh[i][c] = xh;
    s_sc[i][c] = a.score == SPA_SCORE_MAGNITUDE ? __builtin_fabsf(xh) : __builtin_fabsf(xh) * s_f[c];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < T_ * KM; e += 256) {
    const int i = e / KM, c = e % KM, j = c % M, base = c - j;
    if (c >= KV) { s_keep[i][c] = 0; continue; }
    const float me = s_sc[i][c];
    int rank = 0;
#pragma unroll
    for (int q = 0; q < M; ++q) rank += beats(s_sc[i][base + q], q, me, j) ? 1 : 0;
    const bool keep = rank < a.n;
    s_keep[i][c] = keep ? 1 : 0;
    if (keep) atomicOr(&s_tm[c], 1u << i);
  }
  __syncthreads();
  const int kept_row = a.k / M * a.n;
  uint16_t* coef = a.coef;
  for (int e = threadIdx.x; e < kMaxTok * KV; e += 256) {
    const int c = e / kMaxTok, i = e % kMaxTok;
    uint16_t v = 0;
    if (i < T_ && s_keep[i][c]) v = (uint16_t)from_f32<DT>(s_xh[i][c]);
    coef[(size_t)(kb + c) * kMaxTok + i] = v;
    if (i < T_ && s_keep[i][c] && a.idx_out) {
      const int j = c % M, base = c - j;
      int before = 0;
      for (int q = 0; q < j; ++q) before += s_keep[i][base + q];
      a.idx_out[(size_t)i * kept_row + (size_t)(kb + base) / M * a.n + before] = (uint8_t)j;
    }
  }
  if ((int)threadIdx.x < KV) a.tokmask[kb + threadIdx.x] = s_tm[threadIdx.x];
  if (a.var) {
    for (int i = 0; i < T_; ++i) {
      double v0 = 0.0, v1 = 0.0, v2 = 0.0, v3 = 0.0;
      if ((int)threadIdx.x < KV) {
        const int c = threadIdx.x;
        const double v = (double)s_xh[i][c];
        v0 = v; v1 = v * v;
        if (s_keep[i][c]) { v2 = v; v3 = v * v; }
      }
      const double t0 = block_sum(v0, s_red);
      const double t1 = block_sum(v1, s_red);
      const double t2 = block_sum(v2, s_red);
      const double t3 = block_sum(v3, s_red);
      if (threadIdx.x == 0) {
        double* st = a.stats + ((size_t)blockIdx.x * T_ + i) * 4;
        st[0] = t0; st[1] = t1; st[2] = t2; st[3] = t3;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Stream kernel (t > 4): union rows x 128 columns per workgroup on MFMA.
// ---------------------------------------------------------------------------
template <int DT, int MT>
__global__ void __launch_bounds__(256) k_decode_stream(DecodeArgs a) {
  using T = typename Dt<DT>::T;
  constexpr int C = 128;        // columns per workgroup: 4 waves x 2 n-tiles of 16
  constexpr int NT = 2;
  constexpr int KC = 32;        // union rows per MFMA step
  constexpr int WROW = C + 8;   // padded LDS row (halves)
  __shared__ uint16_t s_w[2][KC][WROW];
  __shared__ uint16_t s_a[2][KC][kMaxTok + 2];
  __shared__ int s_rows[256];
  __shared__ int s_cnt[4];
  __shared__ float s_eta[kMaxTok];
  __shared__ float s_nu[kMaxTok];
  __shared__ int s_flag;

  const int T_ = a.t;
  const int tile = blockIdx.x % a.tiles;
  const int split = blockIdx.x / a.tiles;
  const int kb = split * a.k_len;
  const int kend = min(a.k, kb + a.k_len);
  const int c0 = tile * C;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const T* wt = static_cast<const T*>(a.wt);
  const uint16_t* coef = reinterpret_cast<const uint16_t*>(a.coef);

  if ((int)threadIdx.x < T_) s_eta[threadIdx.x] = a.eta ? a.eta[threadIdx.x] : 0.f;

  f32x4 acc[MT][NT];
#pragma unroll
  for (int p = 0; p < MT; ++p)
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[p][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  // W chunk: KC rows x C columns = 32 x 16 segments of 16 bytes -> 2 per thread.
  // Coefficient chunk: KC rows x 64 bytes = 32 x 4 segments -> threads 0..127.
  for (int cb = kb; cb < kend; cb += 256) {
    // union rows of this 256-channel window
    const int c = cb + threadIdx.x;
    const bool f = c < kend && a.tokmask[c] != 0u;
    int U;
    const int pos = block_exclusive_count(f, s_cnt, &U);
    if (f) s_rows[pos] = c;
    __syncthreads();
    const int nchunk = (U + KC - 1) / KC;
    uint4 wreg[2], areg;
    auto load_chunk = [&](int ch) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int sidx = threadIdx.x + 256 * h;
        const int r = sidx >> 4, sg = sidx & 15;
        const int u = ch * KC + r;
        const int colg = c0 + sg * 8;
        if (u < U && colg < a.n_out)
          wreg[h] = *reinterpret_cast<const uint4*>(wt + (size_t)s_rows[u] * a.n_out + colg);
        else
          wreg[h] = make_uint4(0u, 0u, 0u, 0u);
      }
      if (threadIdx.x < 128) {
        const int r = threadIdx.x >> 2, sg = threadIdx.x & 3;
        const int u = ch * KC + r;
        if (u < U)
          areg = *reinterpret_cast<const uint4*>(coef + (size_t)s_rows[u] * kMaxTok + sg * 8);
        else
          areg = make_uint4(0u, 0u, 0u, 0u);
      }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int sidx = threadIdx.x + 256 * h;
        const int r = sidx >> 4, sg = sidx & 15;
        uint32_t* d = reinterpret_cast<uint32_t*>(&s_w[buf][r][sg * 8]);
        d[0] = wreg[h].x; d[1] = wreg[h].y; d[2] = wreg[h].z; d[3] = wreg[h].w;
      }
      if (threadIdx.x < 128) {
        const int r = threadIdx.x >> 2, sg = threadIdx.x & 3;
        uint16_t* d = &s_a[buf][r][sg * 8];
        const uint32_t wds[4] = {areg.x, areg.y, areg.z, areg.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) { d[2 * e] = (uint16_t)(wds[e] & 0xFFFFu); d[2 * e + 1] = (uint16_t)(wds[e] >> 16); }
      }
    };
    if (nchunk > 0) {
      load_chunk(0);
      store_chunk(0);
    }
    __syncthreads();
    for (int ch = 0; ch < nchunk; ++ch) {
      const int buf = ch & 1;
      if (ch + 1 < nchunk) load_chunk(ch + 1);
      // fragments from LDS
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        const int ncol = wv * (NT * 16) + q * 16 + l16;
        uint16_t bh[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bh[j] = s_w[buf][8 * g + j][ncol];
#pragma unroll
        for (int p = 0; p < MT; ++p) {
          uint16_t ah[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) ah[j] = s_a[buf][8 * g + j][16 * p + l16];
          if constexpr (DT == SPA_F16) {
            f16x8 av, bv;
#pragma unroll
            for (int j = 0; j < 8; ++j) { av[j] = __builtin_bit_cast(_Float16, ah[j]); bv[j] = __builtin_bit_cast(_Float16, bh[j]); }
            acc[p][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[p][q], 0, 0, 0);
          } else {
            bf16x8 av, bv;
#pragma unroll
            for (int j = 0; j < 8; ++j) { av[j] = __builtin_bit_cast(__bf16, ah[j]); bv[j] = __builtin_bit_cast(__bf16, bh[j]); }
            acc[p][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[p][q], 0, 0, 0);
          }
        }
      }
      if (ch + 1 < nchunk) store_chunk(buf ^ 1);
      __syncthreads();
    }
  }

  // partial: D lane layout -> token 16p + 4g + r, column l16 of the n-tile
#pragma unroll
  for (int p = 0; p < MT; ++p)
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int col = c0 + wv * (NT * 16) + q * 16 + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = 16 * p + 4 * g + r;
        if (tok < T_ && col < a.n_out) a.partial[((size_t)split * T_ + tok) * a.n_out + col] = acc[p][q][r];
      }
    }
  finish_tile<DT>(a, tile, split, s_eta, &s_flag, s_nu);
}

// ---------------------------------------------------------------------------
// Host planning and launch
// ---------------------------------------------------------------------------
static int pick_splits(int k, int m, int target_splits, int max_k_len) {
  // largest split count <= target with k_len a multiple of m (and of 64 for MFMA windows)
  const int blocks = k / m;
  int s = target_splits < 1 ? 1 : target_splits;
  if (s > blocks) s = blocks;
  int bl = (blocks + s - 1) / s;          // m-blocks per split
  while (bl * m > max_k_len && bl > 1) { ++s; bl = (blocks + s - 1) / s; }
  return bl;
}

size_t decode_workspace(int t, int k, int n_out, int dtype, int n, int m, int score, int shift, int var,
                        DecodeArgs* plan) {
  DecodeArgs p{};
  p.t = t; p.k = k; p.n_out = n_out; p.n = n; p.m = m; p.score = score; p.shift = shift; p.var = var;
  const bool fused = t <= 4 || dtype == SPA_F32;
  size_t bytes = 0;
  auto carve = [&](size_t nbytes) { size_t off = bytes; bytes += (nbytes + 255) & ~(size_t)255; return off; };
  if (fused) {
    const int cpl = dtype == SPA_F32 ? 4 : 8;
    p.col_tile = 64 * cpl;
    p.tiles = (n_out + p.col_tile - 1) / p.col_tile;
    // aim for ~4 workgroups per CU; keep the partial traffic near 5 % of the weight bytes
    int target = (1024 + p.tiles - 1) / p.tiles;
    const double wbytes = (double)k * n / m * n_out * 2.0;
    const int cap = (int)(0.05 * wbytes / (8.0 * t * n_out));
    if (target > cap) target = cap > 1 ? cap : 1;
    // the fused kernel's LDS (scores, coefficients, rows, keep flags, wave partials) stays within 64 KiB
    const int tok = t <= 1 ? 1 : t <= 2 ? 2 : t <= 4 ? 4 : 8;
    int max_kl = (65536 - 16 * tok * p.col_tile) / (4 * (1 + 2 * tok) + tok + 1);
    max_kl = max_kl < 1024 ? max_kl : 1024;
    max_kl = max_kl / 64 * 64;
    if (max_kl < m) max_kl = m;
    const int bl = pick_splits(k, m, target, max_kl);
    p.k_len = bl * m;
    p.splits = (k + p.k_len - 1) / p.k_len;
    p.mask_groups = 0;
    const size_t o_part = carve((size_t)p.splits * t * n_out * 4);
    const size_t o_stats = carve(var ? (size_t)p.tiles * p.splits * t * 4 * 8 : 0);
    const size_t o_cnt = carve((size_t)p.tiles * 4);
    const size_t o_eta = carve((size_t)t * 4);
    p.partial = (float*)o_part; p.stats = (double*)o_stats; p.counters = (unsigned*)o_cnt;
    p.eta_ws = (float*)o_eta;
  } else {
    p.col_tile = 128;
    p.tiles = (n_out + 127) / 128;
    int target = (512 + p.tiles - 1) / p.tiles;
    const int cap = (int)(0.025 * k / t);
    if (target > cap) target = cap > 1 ? cap : 1;
    const int bl = pick_splits(k, 64, target, 1 << 30);
    p.k_len = bl * 64;
    p.splits = (k + p.k_len - 1) / p.k_len;
    p.mask_groups = (k + 63) / 64;
    const size_t o_part = carve((size_t)p.splits * t * n_out * 4);
    const size_t o_stats = carve(var ? (size_t)p.mask_groups * t * 4 * 8 : 0);
    const size_t o_cnt = carve((size_t)p.tiles * 4);
    const size_t o_tm = carve((size_t)k * 4);
    const size_t o_coef = carve((size_t)k * kMaxTok * 2);
    const size_t o_eta = carve((size_t)t * 4);
    p.partial = (float*)o_part; p.stats = (double*)o_stats; p.counters = (unsigned*)o_cnt;
    p.tokmask = (uint32_t*)o_tm; p.coef = (uint16_t*)o_coef; p.eta_ws = (float*)o_eta;
  }
  if (plan) *plan = p;
  return bytes;
}

template <int DT, int M, int TOK>
static hipError_t fused_launch(DecodeArgs& a, hipStream_t st) {
  const int C = a.col_tile;
  const size_t lds = (size_t)a.k_len * 4 * (1 + 2 * TOK) + (((size_t)TOK * a.k_len + 15) & ~(size_t)15) +
                     (size_t)4 * TOK * C * 4;
  hipLaunchKernelGGL((k_decode_fused<DT, M, TOK>), dim3(a.tiles * a.splits), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <int DT, int M>
static hipError_t fused_tok(DecodeArgs& a, hipStream_t st) {
  if (a.t <= 1) return fused_launch<DT, M, 1>(a, st);
  if (a.t <= 2) return fused_launch<DT, M, 2>(a, st);
  if (a.t <= 4) return fused_launch<DT, M, 4>(a, st);
  return fused_launch<DT, M, 8>(a, st);
}

template <int DT>
static hipError_t decode_dt(DecodeArgs& a, hipStream_t st) {
  const bool fused = a.t <= 4 || DT == SPA_F32;
  if (a.shift == SPA_SHIFT_TOKEN_MEAN && (!fused || (size_t)a.t * a.k > 65536)) {
    if (hipError_t e = launch_token_mean(DT, a.x, a.t, a.k, a.eta_ws, st)) return e;
    a.eta = a.eta_ws;
  }
  if (fused) {
    switch (a.m) {
      case 4: return fused_tok<DT, 4>(a, st);
      case 8: return fused_tok<DT, 8>(a, st);
      case 16: return fused_tok<DT, 16>(a, st);
      default: return fused_tok<DT, 32>(a, st);
    }
  }
  if constexpr (DT != SPA_F32) {
    const dim3 mg(a.mask_groups);
    switch (a.m) {
      case 4: hipLaunchKernelGGL((k_decode_mask<DT, 4>), mg, dim3(256), 0, st, a); break;
      case 8: hipLaunchKernelGGL((k_decode_mask<DT, 8>), mg, dim3(256), 0, st, a); break;
      case 16: hipLaunchKernelGGL((k_decode_mask<DT, 16>), mg, dim3(256), 0, st, a); break;
      default: hipLaunchKernelGGL((k_decode_mask<DT, 32>), mg, dim3(256), 0, st, a); break;
    }
    if (hipError_t e = hipGetLastError()) return e;
    if (a.t <= 16)
      hipLaunchKernelGGL((k_decode_stream<DT, 1>), dim3(a.tiles * a.splits), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_decode_stream<DT, 2>), dim3(a.tiles * a.splits), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, DecodeArgs& a, hipStream_t st) {
  switch (dtype) {
    case SPA_F32: return decode_dt<SPA_F32>(a, st);
    case SPA_F16: return decode_dt<SPA_F16>(a, st);
    default: return decode_dt<SPA_BF16>(a, st);
  }
}

}  // namespace spa

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
#include "spa_select.h"

namespace spa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTok = 32;

// ---------------------------------------------------------------------------
// Split-K hand-off without cache-wide maintenance.  A partial is stored with
// agent-scope atomic stores (coherent across the XCDs' private L2s), every
// wave waits for its stores to complete, then one lane takes a ticket with an
// agent-scope atomic.  The last arrival reads the partials back with
// agent-scope atomic loads.  (A device-wide __threadfence() would instead
// write back and invalidate the whole L2 once per workgroup.)
// ---------------------------------------------------------------------------
template <class V>
__device__ __forceinline__ void coherent_store(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class V>
__device__ __forceinline__ V coherent_load(const V* p) {
  return __hip_atomic_load(const_cast<V*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's stores are complete (vmcnt = 0).
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Every thread calls this after its coherent stores; returns true in the
// workgroup that arrives last at this tile.
__device__ __forceinline__ bool arrive_last(unsigned* counter, int expected, int* s_flag) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned ticket = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = ticket == (unsigned)(expected - 1);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// nu from the four per-token sums (sum x, sum x^2, sum kept x, sum kept x^2) over all k.
__device__ __forceinline__ float nu_from_stats(const double* s, int k) {
  const double kk = (double)k;
  const double vf = s[1] / kk - (s[0] / kk) * (s[0] / kk);
  const double vm = s[3] / kk - (s[2] / kk) * (s[2] / kk);
  return vm > 0.0 ? (float)__builtin_sqrt(vf / vm) : 1.f;
}

template <int NW>
__device__ __forceinline__ double wg_sum(double v, double* s_tmp /*[NW]*/) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) s_tmp[w] = v;
  __syncthreads();
  double t = s_tmp[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) t += s_tmp[i];
  return t;
}

// Exclusive prefix sum over the 64 lanes of a wave (Hillis-Steele), *total = sum.
__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
  const int lane = threadIdx.x & 63;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  *total = __shfl(inc, 63, kWave);
  return inc - v;
}

// ---------------------------------------------------------------------------
// Fused variant (t <= TOK).  512 threads = 8 waves.  The workgroup owns C
// columns (8 lanes x one 16-byte load = one 128-byte line of a weight row)
// and a range of channels.  Each thread owns whole m-blocks of the range:
// it shifts and scores its block for every token, selects the top n in
// registers, and lists the block's union rows (with each token's kept value,
// 0 where that token pruned the channel) in a workgroup-shared LDS list.
// All eight waves then stream the listed rows, 8 rows per load instruction,
// and accumulate in float32.
// ---------------------------------------------------------------------------
template <int DT, int M>
__device__ __forceinline__ void load_block(const typename Dt<DT>::T* __restrict__ p, uint4 (&raw)[Dt<DT>::bytes * M / 16 > 0 ? Dt<DT>::bytes * M / 16 : 1]) {
  constexpr int NV = Dt<DT>::bytes * M / 16;
  if constexpr (NV == 0) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);  // 4 x 16-bit
    raw[0] = make_uint4(u.x, u.y, 0u, 0u);
  } else {
#pragma unroll
    for (int q = 0; q < NV; ++q) raw[q] = reinterpret_cast<const uint4*>(p)[q];
  }
}
template <int DT>
__device__ __forceinline__ float raw_elem(const uint4* raw, int j) {
  if constexpr (DT == SPA_F32) {
    const uint4& u = raw[j >> 2];
    const uint32_t w = (j & 3) == 0 ? u.x : (j & 3) == 1 ? u.y : (j & 3) == 2 ? u.z : u.w;
    return __uint_as_float(w);
  } else {
    return elem16<DT>(raw[j >> 3], j & 7);
  }
}

// Waves per workgroup: 8 for the light cases; 4 (so each wave may use up to 512
// registers) when several tokens or 32-wide blocks are ranked per lane.
template <int M, int TOK>
constexpr int fused_waves() { return (TOK >= 2 || M >= 32) ? 4 : 8; }

template <int DT, int M, int TOK>
__global__ void __launch_bounds__((fused_waves<M, TOK>() * 64)) k_decode_fused(DecodeArgs a) {
  using T = typename Dt<DT>::T;
  constexpr int NW = fused_waves<M, TOK>();
  constexpr int NT = NW * 64;
  constexpr int CPL = 16 / Dt<DT>::bytes;                 // columns per 16-byte load
  constexpr int C = 8 * CPL;                              // columns per workgroup
  constexpr int UNR = TOK >= 8 ? 4 : (TOK >= 4 || M >= 32 || DT == SPA_F32) ? 8 : 16;  // loads per batch per lane
  constexpr int NV = Dt<DT>::bytes * M / 16 > 0 ? Dt<DT>::bytes * M / 16 : 1;

  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  __shared__ float s_eta[TOK];
  __shared__ float s_nu[TOK];
  __shared__ double s_red[TOK][NW];
  __shared__ int s_wcnt[NW];
  __shared__ int s_flag;
  __shared__ float s_acc[NW][TOK][C];
  __shared__ double s_st[NW][TOK][4];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int T_ = a.t;
  const int tile = blockIdx.x % a.tiles;
  const int split = blockIdx.x / a.tiles;
  const int c0 = tile * C;
  const int kb = split * a.k_len;
  const int KL = min(a.k_len, a.k - kb);
  const int nb = KL / M;
  const int lcap = a.list_cap;                                       // entries per workgroup
  int* s_rows = reinterpret_cast<int*>(s_dyn);                       // [lcap]
  float* s_coef = reinterpret_cast<float*>(s_dyn) + lcap;            // [TOK][lcap]
  const T* x = static_cast<const T*>(a.x);
  const T* wt = static_cast<const T*>(a.wt);

  // 0. prefetch this thread's first block (every token) and its weight factors
  uint4 raw[TOK][NV];
  float f[M];
#pragma unroll
  for (int j = 0; j < M; ++j) f[j] = 1.f;
  if ((int)threadIdx.x < nb) {
    const int ch0 = kb + (int)threadIdx.x * M;
#pragma unroll
    for (int i = 0; i < TOK; ++i)
      if (i < T_) load_block<DT, M>(x + (size_t)i * a.k + ch0, raw[i]);
    if (a.score == SPA_SCORE_WEIGHT) {
#pragma unroll
      for (int q = 0; q < M / 4; ++q) {
        const float4 v = reinterpret_cast<const float4*>(a.chan_scale + ch0)[q];
        f[4 * q] = v.x; f[4 * q + 1] = v.y; f[4 * q + 2] = v.z; f[4 * q + 3] = v.w;
      }
    }
  }

  // 1. per-token shift: float64 row sums over all k channels (every token at once,
  //    one barrier), fixed reduction order
  if (a.shift == SPA_SHIFT_TOKEN_MEAN && a.eta == nullptr) {
    double sum[TOK];
#pragma unroll
    for (int i = 0; i < TOK; ++i) sum[i] = 0.0;
    const int nq = a.k / CPL;
    for (int q = threadIdx.x; q < nq; q += NT) {
#pragma unroll
      for (int i = 0; i < TOK; ++i) {
        if (i < T_) {
          const uint4 u = *reinterpret_cast<const uint4*>(x + (size_t)i * a.k + (size_t)q * CPL);
          if constexpr (DT == SPA_F32) {
            sum[i] += (double)__uint_as_float(u.x) + (double)__uint_as_float(u.y) + (double)__uint_as_float(u.z) +
                      (double)__uint_as_float(u.w);
          } else {
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) sum[i] += (double)elem16<DT>(u, e2);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < TOK; ++i) {
      const double ws = wave_sum(sum[i]);
      if (lane == 0) s_red[i][wv] = ws;
    }
    __syncthreads();
    if ((int)threadIdx.x < T_) {
      double tot = 0.0;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += s_red[threadIdx.x][w];
      s_eta[threadIdx.x] = (float)(tot / (double)a.k);
    }
  } else if ((int)threadIdx.x < T_) {
    s_eta[threadIdx.x] = a.eta != nullptr ? a.eta[threadIdx.x] : 0.f;
  }
  if (lane == 0)
    for (int i = 0; i < TOK; ++i)
      for (int q = 0; q < 4; ++q) s_st[wv][i][q] = 0.0;
  __syncthreads();
  float eta[TOK];
#pragma unroll
  for (int i = 0; i < TOK; ++i) eta[i] = i < T_ ? s_eta[i] : 0.f;

  // 2. select and list, one block per thread per pass
  const bool write_idx = a.idx_out != nullptr && tile == 0;
  const int kept_row = a.k / M * a.n;
  int base = 0;
  const int npass = (nb + NT - 1) / NT;
  for (int pass = 0; pass < npass; ++pass) {
    const int b = pass * NT + threadIdx.x;
    const bool own = b < nb;
    const int ch0 = kb + b * M;
    if (pass > 0 && own) {
#pragma unroll
      for (int i = 0; i < TOK; ++i)
        if (i < T_) load_block<DT, M>(x + (size_t)i * a.k + ch0, raw[i]);
      if (a.score == SPA_SCORE_WEIGHT) {
#pragma unroll
        for (int j = 0; j < M; ++j) f[j] = a.chan_scale[ch0 + j];
      }
    }
    uint32_t kbits[TOK];
    uint32_t ub = 0;
#pragma unroll
    for (int i = 0; i < TOK; ++i) kbits[i] = 0;
    if (own) {
      if (a.score == SPA_SCORE_CLACT) {
        // column energy over the call's tokens, tokens in order, float32, no FMA
#pragma unroll
        for (int j = 0; j < M; ++j) {
          float acc2 = 0.f;
#pragma unroll
          for (int i = 0; i < TOK; ++i)
            if (i < T_) acc2 = clact_accumulate(acc2, raw_elem<DT>(raw[i], j) - eta[i]);
          f[j] = sqrt_rn(acc2);
        }
      }
#pragma unroll
      for (int i = 0; i < TOK; ++i) {
        if (i < T_) {
          uint32_t sb[M];
#pragma unroll
          for (int j = 0; j < M; ++j) {
            const float ax = __builtin_fabsf(raw_elem<DT>(raw[i], j) - eta[i]);
            sb[j] = __float_as_uint(a.score == SPA_SCORE_MAGNITUDE ? ax : ax * f[j]);
          }
          kbits[i] = topn_keep_bits<M>(sb, a.n);
          ub |= kbits[i];
          if (write_idx) {
            uint8_t* ip = a.idx_out + (size_t)i * kept_row + (size_t)(ch0 / M) * a.n;
            int q = 0;
            for (int j = 0; j < M; ++j)
              if ((kbits[i] >> j) & 1u) ip[q++] = (uint8_t)j;
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // one token's network at a time (register pressure)
      }
    }
    if (a.var) {
      // this pass's per-token sums, added to the wave totals in pass order
#pragma unroll
      for (int i = 0; i < TOK; ++i) {
        if (i < T_) {
          double bs[4] = {0.0, 0.0, 0.0, 0.0};
          if (own) {
            for (int j = 0; j < M; ++j) {
              const double v = (double)(raw_elem<DT>(raw[i], j) - eta[i]);
              const double kv = ((kbits[i] >> j) & 1u) ? v : 0.0;
              bs[0] += v;
              bs[1] += v * v;
              bs[2] += kv;
              bs[3] += kv * kv;
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const double tot = wave_sum(bs[q]);
            if (lane == 0) s_st[wv][i][q] += tot;
          }
        }
      }
    }
    // list slots in block order: with one token every block lists exactly n rows;
    // otherwise an exclusive prefix of the union counts over the workgroup
    int slot, total;
    if (T_ == 1) {
      slot = base + b * a.n;
      total = min(NT, nb - pass * NT) * a.n;
    } else {
      int wtot;
      const int wpos = wave_excl_scan(__builtin_popcount(ub), &wtot);
      if (lane == 0) s_wcnt[wv] = wtot;
      __syncthreads();
      int off = base;
      total = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = s_wcnt[w];
        off += w < wv ? c : 0;
        total += c;
      }
      slot = off + wpos;
    }
    if (own) {
#pragma unroll
      for (int j = 0; j < M; ++j) {
        if ((ub >> j) & 1u) {
          s_rows[slot] = ch0 + j;
#pragma unroll
          for (int i = 0; i < TOK; ++i)
            if (i < T_) s_coef[i * lcap + slot] = ((kbits[i] >> j) & 1u) ? raw_elem<DT>(raw[i], j) - eta[i] : 0.f;
          ++slot;
        }
      }
    }
    base += total;
    __syncthreads();
  }

  // 3. stream the listed rows: row group g covers slots 8g..8g+7; wave w takes groups
  //    w, w+NW, ...; lane (rs, cg) loads slot 8g + rs, columns col..col+CPL; two
  //    batches of UNR loads in flight
  const int L = base;
  const int rs = lane >> 3, cg = lane & 7;
  const int col = c0 + cg * CPL;
  const bool cvalid = col < a.n_out;
  float acc[TOK][CPL];
#pragma unroll
  for (int i = 0; i < TOK; ++i)
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[i][e] = 0.f;
  const int G = (L + 7) / 8;
  uint4 wa[UNR], wb[UNR];
  auto issue = [&](uint4 (&w)[UNR], int it) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int u = ((it * UNR + j) * NW + wv) * 8 + rs;
      if (u < L && cvalid)
        w[j] = *reinterpret_cast<const uint4*>(wt + (size_t)s_rows[u] * a.n_out + col);
      else
        w[j] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto consume = [&](const uint4 (&w)[UNR], int it) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int u = ((it * UNR + j) * NW + wv) * 8 + rs;
      if (u < L) {
        float wf[CPL];
        if constexpr (DT == SPA_F32) {
          wf[0] = __uint_as_float(w[j].x); wf[1] = __uint_as_float(w[j].y);
          wf[2] = __uint_as_float(w[j].z); wf[3] = __uint_as_float(w[j].w);
        } else {
#pragma unroll
          for (int e = 0; e < CPL; ++e) wf[e] = elem16<DT>(w[j], e);
        }
#pragma unroll
        for (int i = 0; i < TOK; ++i) {
          if (i < T_) {
            const float cf = s_coef[i * lcap + u];
#pragma unroll
            for (int e = 0; e < CPL; ++e) acc[i][e] += cf * wf[e];
          }
        }
      }
    }
  };
  const int nit = (G + NW * UNR - 1) / (NW * UNR);   // batches, uniform across the workgroup
  if (nit > 0) issue(wa, 0);
  for (int it = 0; it < nit; it += 2) {
    if (it + 1 < nit) issue(wb, it + 1);
    consume(wa, it);
    if (it + 2 < nit) issue(wa, it + 2);
    if (it + 1 < nit) consume(wb, it + 1);
  }

  // 5. reduce: the 8 row lanes of each column group, then the waves in order
#pragma unroll
  for (int i = 0; i < TOK; ++i)
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      float v = acc[i][e];
      v += __shfl_xor(v, 8, kWave);
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      acc[i][e] = v;
    }
  if (rs == 0) {
#pragma unroll
    for (int i = 0; i < TOK; ++i)
#pragma unroll
      for (int e = 0; e < CPL; ++e) s_acc[wv][i][cg * CPL + e] = acc[i][e];
  }
  __syncthreads();

  const int p = threadIdx.x;            // one (token, column) per thread: T_ * C <= 256
  const int pi = p / C, pc = p % C, pcol = c0 + pc;
  const bool pact = pi < T_ && pcol < a.n_out;
  float v = 0.f;
  if (pact) {
#pragma unroll
    for (int w = 0; w < NW; ++w) v += s_acc[w][pi][pc];
  }
  double stats[4] = {0.0, 0.0, 0.0, 0.0};
  if (a.var && pi < T_ && pc == 0) {
    for (int w = 0; w < NW; ++w)
      for (int q = 0; q < 4; ++q) stats[q] += s_st[w][pi][q];
  }

  if (a.splits > 1) {
    if (pact) coherent_store(&a.partial[((size_t)split * T_ + pi) * a.n_out + pcol], v);
    if (a.var && pi < T_ && pc == 0)
      for (int q = 0; q < 4; ++q)
        coherent_store(&a.stats[(((size_t)tile * a.splits + split) * T_ + pi) * 4 + q], stats[q]);
    if (!arrive_last(&a.counters[tile], a.splits, &s_flag)) return;
    if (pact) {
      // all loads first, then the sum in split order
      v = 0.f;
      for (int s0 = 0; s0 < a.splits; s0 += 16) {
        float part[16];
#pragma unroll
        for (int q = 0; q < 16; ++q)
          part[q] = s0 + q < a.splits ? coherent_load(&a.partial[((size_t)(s0 + q) * T_ + pi) * a.n_out + pcol]) : 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (s0 + q < a.splits) v += part[q];
      }
    }
    if (a.var && pi < T_ && pc == 0) {
      for (int q = 0; q < 4; ++q) stats[q] = 0.0;
      for (int s2 = 0; s2 < a.splits; ++s2)
        for (int q = 0; q < 4; ++q)
          stats[q] += coherent_load(&a.stats[(((size_t)tile * a.splits + s2) * T_ + pi) * 4 + q]);
    }
  }
  // 6. epilogue
  if (pi < T_ && pc == 0) {
    const float nu = a.var ? nu_from_stats(stats, a.k) : 1.f;
    s_nu[pi] = nu;
    if (tile == 0 && a.nu_out) a.nu_out[pi] = nu;
  }
  __syncthreads();
  if (pact) {
    float out = s_nu[pi] * v;
    if (a.shift != SPA_SHIFT_NONE) out += s_eta[pi] * a.row_sum[pcol];
    static_cast<T*>(a.y)[(size_t)pi * a.n_out + pcol] = from_f32<DT>(out);
  }
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
        if (tok < T_ && col < a.n_out)
          coherent_store(&a.partial[((size_t)split * T_ + tok) * a.n_out + col], acc[p][q][r]);
      }
    }
  if (!arrive_last(&a.counters[tile], a.splits, &s_flag)) return;

  // last workgroup of the tile: nu from the mask kernel's per-group sums, then y
  if ((int)threadIdx.x < T_) {
    float nu = 1.f;
    if (a.var) {
      double st[4] = {0.0, 0.0, 0.0, 0.0};
      for (int g2 = 0; g2 < a.mask_groups; ++g2)
        for (int q = 0; q < 4; ++q) st[q] += a.stats[((size_t)g2 * T_ + threadIdx.x) * 4 + q];
      nu = nu_from_stats(st, a.k);
    }
    s_nu[threadIdx.x] = nu;
    if (tile == 0 && a.nu_out) a.nu_out[threadIdx.x] = nu;
  }
  __syncthreads();
  T* y = static_cast<T*>(a.y);
  const int cw = min(C, a.n_out - c0);
  for (int pidx = threadIdx.x; pidx < T_ * cw; pidx += 256) {
    const int tok = pidx / cw, col = c0 + pidx % cw;
    float v = 0.f;
    for (int s0 = 0; s0 < a.splits; s0 += 16) {
      float part[16];
#pragma unroll
      for (int q = 0; q < 16; ++q)
        part[q] = s0 + q < a.splits ? coherent_load(&a.partial[((size_t)(s0 + q) * T_ + tok) * a.n_out + col]) : 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (s0 + q < a.splits) v += part[q];
    }
    float out = s_nu[tok] * v;
    if (a.shift != SPA_SHIFT_NONE) out += s_eta[tok] * a.row_sum[col];
    y[(size_t)tok * a.n_out + col] = from_f32<DT>(out);
  }
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
    // 8 lanes x one 16-byte load = one 128-byte cache line of every listed row
    const int cpl = dtype == SPA_F32 ? 4 : 8;
    p.col_tile = 8 * cpl;
    p.tiles = (n_out + p.col_tile - 1) / p.col_tile;
    // split the channels only when the column tiles alone cannot fill the 256 CUs;
    // each wave keeps at least one block, and the partial traffic stays near 5 % of the weight bytes
    const int blocks = k / m;
    int sp = p.tiles >= 192 ? 1 : (256 + p.tiles - 1) / p.tiles;
    const int max_by_waves = blocks / 8 > 1 ? blocks / 8 : 1;
    const double wbytes = (double)k * n / m * n_out * 2.0;
    const int max_by_traffic = (int)(0.05 * wbytes / (8.0 * t * n_out));
    if (sp > max_by_waves) sp = max_by_waves;
    if (sp > max_by_traffic) sp = max_by_traffic > 1 ? max_by_traffic : 1;
    // the workgroup's row list (row index + one coefficient per token per entry) lives in LDS:
    // at most 54 KiB
    const int tok = t <= 1 ? 1 : t <= 2 ? 2 : t <= 4 ? 4 : 8;
    const int per_block = m < n * t ? m : n * t;          // union rows one block can contribute
    const int max_entries = 55296 / (4 * (1 + tok));
    const int max_blocks = max_entries / per_block > 1 ? max_entries / per_block : 1;
    int bl = (blocks + sp - 1) / sp;
    if (bl > max_blocks) bl = max_blocks;
    p.k_len = bl * m;
    p.splits = (k + p.k_len - 1) / p.k_len;
    p.list_cap = bl * per_block;
    p.chunk_blocks = bl;
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
  constexpr int NW = fused_waves<M, TOK>();
  const size_t lds = (size_t)a.list_cap * 4 * (1 + TOK);
  hipLaunchKernelGGL((k_decode_fused<DT, M, TOK>), dim3(a.tiles * a.splits), dim3(NW * 64), lds, st, a);
  return hipGetLastError();
}

template <int DT, int M>
static hipError_t fused_tok(DecodeArgs& a, hipStream_t st) {
  if (a.t <= 1) return fused_launch<DT, M, 1>(a, st);
  if (a.t <= 2) return fused_launch<DT, M, 2>(a, st);
  if (a.t <= 4) return fused_launch<DT, M, 4>(a, st);
  if constexpr (DT == SPA_F32) return fused_launch<DT, M, 8>(a, st);  // 16-bit t > 4 takes the MFMA path
  return hipErrorInvalidValue;
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

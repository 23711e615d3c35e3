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
// Variants:
//  * one token, 16-bit weights under 2 GiB, at least eight 512-column tiles
//    (k_decode_t1): each wave forms the shift itself, selects its own 64
//    channels at a time by in-block rank and streams their kept rows, 1 KB
//    of a row per load, 32 buffer loads per lane in flight, with no
//    workgroup barrier before the stream;
//  * fused (float32 up to 8 tokens, and one 16-bit token with narrower
//    outputs or a weight of 2 GiB or more): each workgroup prunes its own
//    channel range in LDS (the same few thousand comparisons in every tile)
//    and streams the union of kept rows with float32 VALU FMAs, 16 bytes per
//    lane per row;
//  * matrix-core (2..32 tokens, 16-bit): the union of kept rows is most or
//    nearly all of W (three quarters at two tokens of 8:16), so k_prune_cols
//    prunes every channel once into masked rows in the matrix cores' operand
//    order, and k_decode_mm reads the row-major W once
//    and runs the product on matrix cores (mfma 16x16x32).
#include "spa_common.h"
#include "spa_launch.h"
#include "spa_plan.h"
#include "spa_select.h"

namespace spa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTok = 32;

// Loads of the weight streams carry the non-temporal hint: each weight row is
// read once per call, so its lines need not displace reused data in L2 or
// the MALL.  kCacheNonTemporal is the buffer-load cache-policy value of the
// nt bit on gfx950.
constexpr int kCacheNonTemporal = 2;
__device__ __forceinline__ void lds_dma16_nt(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(sbase), "s"(lds)
               : "m0");
}

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
__device__ __forceinline__ float nu_from_stats(const double* s, const DecodeArgs& a, int tok, bool writer) {
  const double kk = (double)a.k;
  const double vf = s[1] / kk - (s[0] / kk) * (s[0] / kk);
  const double vm = s[3] / kk - (s[2] / kk) * (s[2] / kk);
  return nu_of(vf, vm, a.var, a.var_in, a.var_out, tok, writer);
}

// Sum over the splits of a tile, in split order, of entry `e` of each split's
// float64 block (blocks `stride` apart): all loads in flight before the adds.
__device__ __forceinline__ double split_sum_f64(const double* base, int splits, int stride, int e) {
  double acc = 0.0;
  for (int s0 = 0; s0 < splits; s0 += 16) {
    double part[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
      part[q] = s0 + q < splits ? coherent_load(base + (size_t)(s0 + q) * stride + e) : 0.0;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (s0 + q < splits) acc += part[q];
  }
  return acc;
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

// The squared-ReLU input transform applied in place to raw words (16-bit
// halves or float32 words).  Its results are representable in the dtype, so
// the words stay exact.
template <int DT, int NQ>
__device__ __forceinline__ void act_raw(uint4 (&raw)[NQ]) {
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    uint32_t* w = reinterpret_cast<uint32_t*>(&raw[q]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (DT == SPA_F32) {
        w[e] = __float_as_uint(relu2<DT>(__uint_as_float(w[e])));
      } else {
        const uint32_t lo = (uint32_t)from_f32<DT>(relu2<DT>(to_f32<DT>((uint16_t)(w[e] & 0xFFFFu))));
        const uint32_t hi = (uint32_t)from_f32<DT>(relu2<DT>(to_f32<DT>((uint16_t)(w[e] >> 16))));
        w[e] = lo | (hi << 16);
      }
    }
  }
}

template <int M, int TOK>
constexpr int fused_waves() { return fused_waves_of(M, TOK); }

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
  __shared__ double s_stsum[TOK * 4];

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
            sum[i] += (double)apply_act<DT>(__uint_as_float(u.x), a.act) +
                      (double)apply_act<DT>(__uint_as_float(u.y), a.act) +
                      (double)apply_act<DT>(__uint_as_float(u.z), a.act) +
                      (double)apply_act<DT>(__uint_as_float(u.w), a.act);
          } else {
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) sum[i] += (double)apply_act<DT>(elem16<DT>(u, e2), a.act);
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
    if (a.act && own) {
#pragma unroll
      for (int i = 0; i < TOK; ++i)
        if (i < T_) act_raw<DT>(raw[i]);
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
      slot = one_token_list_slot(base, (int)threadIdx.x, a.n);
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
    if (a.var) {   // one thread per (token, sum), every split's value in flight at once
      if ((int)threadIdx.x < T_ * 4)
        s_stsum[threadIdx.x] = split_sum_f64(a.stats + (size_t)tile * a.splits * T_ * 4, a.splits, T_ * 4, threadIdx.x);
      __syncthreads();
      if (pi < T_ && pc == 0)
        for (int q = 0; q < 4; ++q) stats[q] = s_stsum[pi * 4 + q];
    }
  }
  // 6. epilogue
  if (pi < T_ && pc == 0) {
    const float nu = a.var ? nu_from_stats(stats, a, pi, tile == 0) : 1.f;
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
// One token, 16-bit weights, wide outputs (the latency-critical GEMV).
//   * Work split: workgroup (tile, split) owns 512 columns and a channel range
//     of at most kT1MaxChan channels; a load instruction reads 1 KB of one
//     weight row (long runs per row stream HBM faster than eight 128-byte
//     pieces of eight rows).  Splits hand off through the ticket above.
//   * The mean shift: every wave sums the whole token row in float64 (eight
//     16-byte loads per lane per 4096 channels in flight, then a fixed-order
//     wave sum), so no workgroup barrier precedes the stream.
//   * Each wave then works alone on 64 channels at a time: a lane scores its
//     channel, counts the positions of its m-block that beat it (larger
//     score, or equal score at a lower position) -- by 64-bit rank keys read
//     back from the wave's LDS slots for m <= 16, by xor swizzles inside the
//     block for m = 32 -- and keeps the channel when fewer than n do.  A ballot orders the
//     wave's kept channels; their (row, coefficient) pairs pass through the
//     wave's own LDS slots, and the wave streams exactly those rows, up to
//     kT1Loads loads per lane in flight, row offsets and coefficients held in
//     scalar registers.  No wave waits for another before its stream.
// ---------------------------------------------------------------------------
constexpr int kT1Loads = 32;
static_assert(kPlanBufferLimit == kBufferOutOfRange, "one buffer limit");

// so[q] = v of lane (lane ^ q), q = 1 .. M-1, inside groups of 32 lanes
// (ds_swizzle bit mode: and-mask 31, xor-mask q).
template <int M, int Q = 1>
__device__ __forceinline__ void swizzle_xor_all(uint32_t v, uint32_t (&so)[M]) {
  if constexpr (Q < M) {
    so[Q] = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (Q << 10));
    swizzle_xor_all<M, Q + 1>(v, so);
  }
}

// ACT: the squared-ReLU input transform, a template switch so that the plain
// kernel's code is not touched by it.
template <int DT, int M, bool ACT>
__global__ void __launch_bounds__(kT1Threads) k_decode_t1(DecodeArgs a) {
  using T = typename Dt<DT>::T;
  constexpr int NW = kT1Waves, NT = kT1Threads, CPL = 8, C = kT1Cols;
  constexpr int R = kT1MaxChan / NT;                       // channel rounds per thread
  static_assert(64 % M == 0 && M <= 32, "an m-block must sit inside one wave");
  __shared__ float s_acc[NW][C];
  __shared__ __attribute__((aligned(16))) uint2 s_ent[NW][64];   // per wave: (row, coefficient bits) of its kept channels
  __shared__ __attribute__((aligned(16))) unsigned long long s_key[NW][64];   // per wave: the round's rank keys
  __shared__ double s_part[NW][5];                         // row-sum partial, then the four variance sums
  __shared__ double s_stsum[4];
  __shared__ float s_nu;
  __shared__ int s_flag;

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int tile = blockIdx.x % a.tiles, split = blockIdx.x / a.tiles;
  const int c0 = tile * C;
  const int kb = split * a.k_len;
  const int KL = min(a.k_len, a.k - kb);                   // a multiple of M, <= kT1MaxChan
  const T* x = static_cast<const T*>(a.x);
  const T* wt = static_cast<const T*>(a.wt);

  // 0. this thread's channels (and their factors), then its share of the row
  //    for the mean: buffer loads, all issued before anything waits (offsets
  //    past the end read zeros, so no load sits under a branch)
  const bool wscore = a.score == SPA_SCORE_WEIGHT;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(x), (short)0, a.k * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
      wscore ? (void*)a.chan_scale : const_cast<T*>(x), (short)0, wscore ? a.k * 4 : 0, kBufferWord3);
  uint32_t xraw[R], fraw[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = NT * r + threadIdx.x;
    xraw[r] = buffer_load_u16(xr, c < KL ? (uint32_t)(kb + c) * 2u : kBufferOutOfRange);
    fraw[r] = buffer_load_u32(fr, c < KL ? (uint32_t)(kb + c) * 4u : kBufferOutOfRange);
  }
  // 1. the shift: every wave sums the whole row itself (the same loads and
  //    the same fixed order in every wave and workgroup, so every wave forms
  //    the same eta), with no workgroup barrier: a wave goes on to its rows
  //    as soon as its own loads are back
  const bool mean = a.shift == SPA_SHIFT_TOKEN_MEAN && a.eta == nullptr;
  float eta = 0.f;
  if (mean) {
    const int nq = a.k / 8;                                // 16-byte pieces of the row
    double part[4] = {0.0, 0.0, 0.0, 0.0};
    for (int q0 = 0; q0 < nq; q0 += 8 * 64) {
      uint4 u[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = q0 + 64 * i + lane;
        u[i] = buffer_load16(xr, q < nq ? (uint32_t)q * 16u : kBufferOutOfRange);
      }
      // every load issued before the first use (the scheduler would otherwise
      // start the sums on the first piece and wait for it, all loads
      // outstanding, before issuing the other seven: two round trips)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) part[i & 3] += (double)apply_act<DT>(elem16<DT>(u[i], e), ACT);
    }
    const double tot = wave_sum_dpp((part[0] + part[1]) + (part[2] + part[3]));
    eta = (float)(tot / (double)a.k);
  } else if (a.eta != nullptr) {
    eta = a.eta[0];
  }

  const uint32_t wt_bytes = (uint32_t)a.k * (uint32_t)a.n_out * 2u;
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(wt), (short)0,
                                                                          (int)wt_bytes, kBufferWord3);
  const uint32_t col_bytes = (uint32_t)min(c0 + lane * CPL, a.n_out - CPL) * 2u;   // lanes past n_out: never stored
  const uint32_t row_bytes = (uint32_t)a.n_out * 2u;
  const int j = lane % M;
  float acc[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) acc[e] = 0.f;
  double st[4] = {0.0, 0.0, 0.0, 0.0};

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int cw = NT * r + 64 * wv;                       // this wave's first channel of the round
    if (cw >= KL) break;                                   // uniform
    const int c = cw + lane;
    // 2. score (one loop per score kind under a uniform branch: if-converted,
    //    every kind would pay for CLACT's square root)
    const float xh = apply_act<DT>(to_f32<DT>((T)xraw[r]), ACT) - eta;
    uint32_t sb;
    if (a.score == SPA_SCORE_MAGNITUDE) {
      sb = __float_as_uint(__builtin_fabsf(xh));
    } else if (a.score == SPA_SCORE_WEIGHT) {
      sb = __float_as_uint(__builtin_fabsf(xh) * __uint_as_float(fraw[r]));
    } else {                                               // one token: the column energy is the square alone
      sb = __float_as_uint(__builtin_fabsf(xh) * sqrt_rn(clact_accumulate(0.f, xh)));
    }
    // 3. rank inside the block; scores are non-negative floats, so their bit
    //    patterns order like the values and stay below 2^31
    int beat = 0;
    if constexpr (M <= 16) {
      // by 64-bit keys (score bits, 31 - position): a larger key is a larger
      // score or an equal score at a lower position.  The wave parks its
      // keys in its own LDS slots and reads its block's back as broadcast
      // 16-byte reads (the wave's LDS operations run in order); one compare
      // per block member (17.07 -> 16.91 us at the decode layer, alternating runs)
      const unsigned long long key = ((unsigned long long)sb << 32) | (uint32_t)(31 - j);
      s_key[wv][lane] = key;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int q = 0; q < M / 2; ++q) {
        const uint4 v = *reinterpret_cast<const uint4*>(&s_key[wv][lane - j + 2 * q]);
        beat += (((unsigned long long)v.y << 32) | v.x) > key ? 1 : 0;
        beat += (((unsigned long long)v.w << 32) | v.z) > key ? 1 : 0;
      }
    } else {
      // 32-wide blocks: xor swizzles inside 32-lane groups, all issued before
      // the first compare; adding 1 for a lower position turns "greater or
      // equal" into "greater" (the keys above measured 19.19 -> 19.64 us here)
      uint32_t so[M];
      swizzle_xor_all<M>(sb, so);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 1; q < M; ++q) beat += (so[q] + ((j ^ q) < j ? 1u : 0u)) > sb ? 1 : 0;
    }
    const bool keep = c < KL && beat < a.n;
    const unsigned long long kmask = __ballot(keep);
    const int cnt = __popcll(kmask);                        // uniform
    const int slot = __popcll(kmask & ((1ull << lane) - 1ull));
    if (keep) {
      s_ent[wv][slot] = make_uint2((uint32_t)(kb + c), __float_as_uint(xh));
      if (a.idx_out != nullptr && tile == 0)
        a.idx_out[(size_t)(kb + c - j) / M * a.n + (slot - (lane / M) * a.n)] = (uint8_t)j;
    }
    if (a.var && c < KL) {
      const double v = (double)xh;
      st[0] += v;
      st[1] += v * v;
      if (keep) { st[2] += v; st[3] += v * v; }
    }
    // the wave's LDS writes are complete before its reads (one wave, in order)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 4. stream the wave's kept rows, kT1Loads at a time.  For m <= 16 every
    //    lane reads the batch's entries itself (broadcast LDS reads, two
    //    entries each), so row offsets and coefficients sit in vector
    //    registers; as scalars (read lane by lane) 64 of them per batch
    //    spilled to vector lanes and back.  32-wide blocks keep the scalar
    //    form: their swizzled rank already fills the vector registers.
    const uint2 mine = s_ent[wv][lane];                    // entry `lane` (stale past cnt, never used)
    for (int b0 = 0; b0 < cnt; b0 += kT1Loads) {
      uint32_t soff[kT1Loads], voff[kT1Loads];
      float cf[kT1Loads];
      if constexpr (M <= 16) {
#pragma unroll
        for (int i = 0; i < kT1Loads; i += 2) {
          const uint4 pr = *reinterpret_cast<const uint4*>(&s_ent[wv][(b0 + i) & 63]);   // entries b0 + i, + 1
          const bool ok0 = b0 + i < cnt, ok1 = b0 + i + 1 < cnt;   // uniform
          soff[i] = soff[i + 1] = 0u;
          voff[i] = ok0 ? pr.x * row_bytes + col_bytes : kBufferOutOfRange;
          cf[i] = ok0 ? __uint_as_float(pr.y) : 0.f;
          voff[i + 1] = ok1 ? pr.z * row_bytes + col_bytes : kBufferOutOfRange;
          cf[i + 1] = ok1 ? __uint_as_float(pr.w) : 0.f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < kT1Loads; ++i) {
          const int e = b0 + i;
          const bool ok = e < cnt;                           // uniform
          const uint32_t row = (uint32_t)__builtin_amdgcn_readlane((int)mine.x, e & 63);
          soff[i] = ok ? row * row_bytes : 0u;
          voff[i] = ok ? col_bytes : kBufferOutOfRange;
          cf[i] = ok ? __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)mine.y, e & 63)) : 0.f;
        }
      }
      uint4 w[kT1Loads];
#pragma unroll
      for (int i = 0; i < kT1Loads; ++i) {
        // non-temporal: each kept row is read once per call
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)voff[i], (int)soff[i], kCacheNonTemporal);
        w[i] = make_uint4(v[0], v[1], v[2], v[3]);
      }
      __builtin_amdgcn_sched_barrier(0);                   // every load issued before the first use
#pragma unroll
      for (int i = 0; i < kT1Loads; ++i) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) acc[e] += cf[i] * elem16<DT>(w[i], e);
      }
    }
  }
  // 5. the waves in order
  if (a.var) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double tot = wave_sum_dpp(st[q]);
      if (lane == 0) s_part[wv][1 + q] = tot;
    }
  }
#pragma unroll
  for (int e = 0; e < CPL; ++e) s_acc[wv][lane * CPL + e] = acc[e];
  __syncthreads();
  const int pc = threadIdx.x, pcol = c0 + pc;
  const bool pact = pcol < a.n_out;
  const float rsum = (pact && a.shift != SPA_SHIFT_NONE) ? a.row_sum[pcol] : 0.f;
  float v = 0.f;
  if (pact) {
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) v += s_acc[w2][pc];
  }
  double stats[4] = {0.0, 0.0, 0.0, 0.0};
  if (a.var && threadIdx.x == 0)
    for (int w2 = 0; w2 < NW; ++w2)
      for (int q = 0; q < 4; ++q) stats[q] += s_part[w2][1 + q];
  if (a.splits > 1) {
    if (pact) coherent_store(&a.partial[(size_t)split * a.n_out + pcol], v);
    if (a.var && threadIdx.x == 0)
      for (int q = 0; q < 4; ++q) coherent_store(&a.stats[((size_t)tile * a.splits + split) * 4 + q], stats[q]);
    if (!arrive_last(&a.counters[tile], a.splits, &s_flag)) return;
    if (pact) {
      v = 0.f;
      for (int s0 = 0; s0 < a.splits; s0 += 16) {
        float part[16];
#pragma unroll
        for (int q = 0; q < 16; ++q)
          part[q] = s0 + q < a.splits ? coherent_load(&a.partial[(size_t)(s0 + q) * a.n_out + pcol]) : 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (s0 + q < a.splits) v += part[q];
      }
    }
    if (a.var) {   // one thread per sum, every split's value in flight at once
      if (threadIdx.x < 4) s_stsum[threadIdx.x] = split_sum_f64(a.stats + (size_t)tile * a.splits * 4, a.splits, 4, threadIdx.x);
      __syncthreads();
      if (threadIdx.x == 0)
        for (int q = 0; q < 4; ++q) stats[q] = s_stsum[q];
    }
  }
  // 6. epilogue
  if (threadIdx.x == 0) {
    const float nu = a.var ? nu_from_stats(stats, a, 0, tile == 0) : 1.f;
    s_nu = nu;
    if (tile == 0 && a.nu_out) a.nu_out[0] = nu;
  }
  __syncthreads();
  if (pact) {
    float out = s_nu * v;
    if (a.shift != SPA_SHIFT_NONE) out += eta * rsum;
    static_cast<T*>(a.y)[pcol] = from_f32<DT>(out);
  }
}

// ---------------------------------------------------------------------------
// Pruning pass of the matrix-core decode (t >= 2): few token rows, so the
// work is cut by channels and by token.  Workgroup (chunk, quarter) owns
// kPruneChan channels and the tokens quarter, quarter + 4, ...: it stages
// x_hat = x - eta of its channels for every token in LDS (each thread one
// channel of eight tokens, all of its loads in flight), since the CLACT
// column energy needs every token of a channel.  16 waves: wave w owns the 64
// channels 64 (w % 4) .. +63 of the chunk, one per lane, and the quarter's
// tokens w / 4 and w / 4 + 4 (two tokens of serial work per wave).  A lane
// forms its channel factor, and for each of its tokens scores its channel,
// parks the score in the wave's LDS slots, reads its m-block's scores back
// (broadcast 16-byte reads) and keeps the channel when fewer than n of them
// beat it (larger, or equal at a lower position).  It writes the masked
// values, the kept positions and each token's four variance sums of the
// chunk (the four channel groups added in order); the matrix-core pass
// folds the chunks into nu.
//
// The masked activations are written in the GEMM's operand order ("fragment
// order"): for 64-channel step s, token block tb (16 tokens) and window h,
// one 1 KB run where lane d = m + 16 g holds channels 64 s + 16 g + 8 h .. +7
// of token 16 tb + m.  Token lanes past t, and channel groups past k, are
// never written or read.
// ---------------------------------------------------------------------------
constexpr int kPcThreads = 1024;

// The value of lane (lane ^ K) of the wave: DPP for K = 1, 2 (quad
// permutes) and 8 (a rotation by 8 inside each row of 16 lanes), a swizzle
// inside each half-wave for K = 4 and 16, an LDS permute for K = 32.
template <int K>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v) {
  if constexpr (K == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
  else if constexpr (K == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
  else if constexpr (K == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);
  else if constexpr (K == 32)
    return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((threadIdx.x & 63) ^ 32) * 4), (int)v);
  else return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (K << 10));
}
template <int K>
__device__ __forceinline__ double lane_xor_f64(double d) {
  const uint64_t u = __builtin_bit_cast(uint64_t, d);
  const uint32_t lo = lane_xor_u32<K>((uint32_t)u), hi = lane_xor_u32<K>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ size_t frag_offset(int step, int tb, int ntb, int h, int lane) {
  return ((((size_t)step * ntb + tb) * 2 + h) * 64 + lane) * 8;   // in 16-bit elements
}

template <int DT, int M>
__global__ void __launch_bounds__(kPcThreads) k_prune_cols(DecodeArgs a) {
  using T = typename Dt<DT>::T;
  constexpr int CH = kPruneChan, NW = kPcThreads / 64;
  static_assert(CH == 256 && NW == 16, "four waves per 64-channel group, one channel per lane");
  __shared__ __attribute__((aligned(16))) float s_x[kMaxTok][CH];
  __shared__ __attribute__((aligned(16))) unsigned long long s_sc[NW][64];   // per wave: the current token's rank keys
  __shared__ __attribute__((aligned(16))) uint16_t s_mv[NW][64];   // per wave: its masked values
  __shared__ double s_st[4][kMaxTok / 4][4];
  const int T_ = a.t, K = a.k;
  const int ntb = (T_ + 15) / 16;
  const int c0 = blockIdx.x * CH, quarter = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // The token means, when this pass forms them (short calls, t k <= 65536; a
  // separate pass otherwise): every workgroup sums every token row itself,
  // wave w rows w, w + 16, ...: float64 over 16-byte loads (eight per lane in
  // flight), then a fixed butterfly over the lanes.  Workgroup (0, 0) leaves
  // the means in the workspace for the product's epilogue.
  __shared__ float s_eta[kMaxTok];
  const bool own_mean = a.shift == SPA_SHIFT_TOKEN_MEAN && a.eta == nullptr;
  if (own_mean) {
    const int nq = K / 8;                                   // k % 16 == 0: whole 16-byte pieces
    for (int i = wv; i < T_; i += NW) {
      const uint4* row = reinterpret_cast<const uint4*>(static_cast<const T*>(a.x) + (size_t)i * K);
      double part = 0.0;
      for (int q0 = 0; q0 < nq; q0 += 8 * 64) {
        uint4 u[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int q = q0 + 64 * r + lane;
          u[r] = q < nq ? row[q] : make_uint4(0u, 0u, 0u, 0u);   // zeros add nothing (also squared)
        }
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) part += (double)apply_act<DT>(elem16<DT>(u[r], e), a.act);
      }
      part += lane_xor_f64<1>(part);
      part += lane_xor_f64<2>(part);
      part += lane_xor_f64<4>(part);
      part += lane_xor_f64<8>(part);
      part += lane_xor_f64<16>(part);
      part += lane_xor_f64<32>(part);
      if (lane == 0) s_eta[i] = (float)(part / (double)K);
    }
    __syncthreads();
    if (blockIdx.x == 0 && blockIdx.y == 0 && (int)threadIdx.x < T_) a.eta_ws[threadIdx.x] = s_eta[threadIdx.x];
  }
  {
    // thread (i, p) stages channels c0 + 8 p .. + 7 of token i = thread / 32
    // with one 16-byte buffer load (offsets past the end read zeros); rows
    // past t, and channels past k, are zero
    const int i = threadIdx.x >> 5, p = threadIdx.x & 31, ch = c0 + 8 * p;
    static_assert(kPcThreads == kMaxTok * CH / 8, "one 16-byte piece per thread");
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.x), (short)0, T_ * K * 2, kBufferWord3);
    const bool in = i < T_ && ch < K;                       // k % 16 == 0: a piece is wholly in or out
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, in ? (int)((uint32_t)(i * K + ch) * 2u) : (int)kBufferOutOfRange, 0, 0);
    const float eta = i >= T_ ? 0.f : own_mean ? s_eta[i] : a.eta != nullptr ? a.eta[i] : 0.f;
    const uint4 u = make_uint4(v[0], v[1], v[2], v[3]);
    float xs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xs[e] = in ? apply_act<DT>(elem16<DT>(u, e), a.act) - eta : 0.f;
    *reinterpret_cast<float4*>(&s_x[i][8 * p]) = make_float4(xs[0], xs[1], xs[2], xs[3]);
    *reinterpret_cast<float4*>(&s_x[i][8 * p + 4]) = make_float4(xs[4], xs[5], xs[6], xs[7]);
  }
  __syncthreads();
  // this lane's channel (wave w: group w % 4) and its factor
  const int cg = wv & 3, tw = wv >> 2;
  const int c = 64 * cg + lane, ch = c0 + c;
  const bool cin = ch < K;
  float f = 1.f;
  if (a.score == SPA_SCORE_WEIGHT) {
    f = cin ? a.chan_scale[ch] : 0.f;
  } else if (a.score == SPA_SCORE_CLACT) {
    // column energy over the call's tokens, tokens in order; the zero rows
    // past t add exactly nothing
    float acc = 0.f;
#pragma unroll 8
    for (int i = 0; i < T_; ++i) acc = clact_accumulate(acc, s_x[i][c]);
    f = sqrt_rn(acc);
  }
  const int j = lane % M, b0 = lane - j;                   // position in the block, its first lane
  const int step = (c0 + 64 * cg) / 64;                     // the group's 64 channels are one step
  const int kept_row = K / M * a.n;
  uint16_t* xf = static_cast<uint16_t*>(a.dense);
  // tokens quarter + 4 sl of the quarter's slots sl = tw, tw + 4; this lane's
  // four variance terms of slot u in pv[4 u + q]
  double pv[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sl = tw + 4 * u, i = quarter + 4 * sl;
    if (i >= T_) break;                                     // uniform
    const float xh = s_x[i][c];
    const float ax = __builtin_fabsf(xh);
    const uint32_t sb = __float_as_uint(a.score == SPA_SCORE_MAGNITUDE ? ax : ax * f);
    // rank inside the block by 64-bit keys (score bits, 31 - position):
    // scores are non-negative floats, so their bit patterns order like the
    // values, and a larger key is a larger score or an equal score at a
    // lower position; one compare per block member.  The wave's own LDS
    // writes precede its reads (LDS operations of one wave run in order).
    const unsigned long long key = ((unsigned long long)sb << 32) | (uint32_t)(31 - j);
    s_sc[wv][lane] = key;
    __builtin_amdgcn_wave_barrier();
    unsigned long long sc[M];
#pragma unroll
    for (int q = 0; q < M / 2; ++q) {
      const uint4 v = *reinterpret_cast<const uint4*>(&s_sc[wv][b0 + 2 * q]);
      sc[2 * q] = ((unsigned long long)v.y << 32) | v.x;
      sc[2 * q + 1] = ((unsigned long long)v.w << 32) | v.z;
    }
    int beat = 0;
#pragma unroll
    for (int q = 0; q < M; ++q) beat += sc[q] > key ? 1 : 0;
    const bool keep = cin && beat < a.n;
    // masked values: eight lanes' values are one 16-byte piece of the operand
    s_mv[wv][lane] = keep ? (uint16_t)from_f32<DT>(xh) : (uint16_t)0;
    __builtin_amdgcn_wave_barrier();
    if (lane < 8 && c0 + 64 * cg + 8 * lane < K) {
      const uint4 v = *reinterpret_cast<const uint4*>(&s_mv[wv][8 * lane]);
      *reinterpret_cast<uint4*>(xf + frag_offset(step, i >> 4, ntb, lane & 1, (i & 15) + 16 * (lane >> 1))) = v;
    }
    if (a.idx_out != nullptr) {
      const unsigned long long km = __ballot(keep);
      const unsigned long long blk = (km >> b0) & ((1ull << M) - 1ull);
      if (keep) {
        const int r = __popcll(blk & ((1ull << j) - 1ull));
        a.idx_out[(size_t)i * kept_row + (size_t)((ch - j) / M) * a.n + r] = (uint8_t)j;
      }
    }
    if (a.var) {
      const double v = (double)xh;                          // 0 past k
      const double kv = keep ? v : 0.0;
      pv[4 * u] = v;
      pv[4 * u + 1] = v * v;
      pv[4 * u + 2] = kv;
      pv[4 * u + 3] = kv * kv;
    }
  }
  if (a.var && quarter + 4 * tw < T_) {                     // the wave has at least one token (uniform)
    // the eight sums over the wave's 64 lanes, in a fixed order: lanes
    // halve the set of sums they carry at each of the first three
    // exchanges (partners lane ^ 1, ^ 2, ^ 4), then the remaining sum is
    // added over lanes ^ 8, ^ 16, ^ 32; lane L < 8 ends with sum
    // 4 (L & 1) + 2 ((L >> 1) & 1) + ((L >> 2) & 1)
    const int p0 = lane & 1, p1 = (lane >> 1) & 1, p2 = (lane >> 2) & 1;
    double w4[4], w2[2];
#pragma unroll
    for (int e = 0; e < 4; ++e) w4[e] = (p0 ? pv[4 + e] : pv[e]) + lane_xor_f64<1>(p0 ? pv[e] : pv[4 + e]);
#pragma unroll
    for (int e = 0; e < 2; ++e) w2[e] = (p1 ? w4[2 + e] : w4[e]) + lane_xor_f64<2>(p1 ? w4[e] : w4[2 + e]);
    double r = (p2 ? w2[1] : w2[0]) + lane_xor_f64<4>(p2 ? w2[0] : w2[1]);
    r += lane_xor_f64<8>(r);
    r += lane_xor_f64<16>(r);
    r += lane_xor_f64<32>(r);
    const int idx = 4 * p0 + 2 * p1 + p2, sl = tw + 4 * (idx >> 2);
    if (lane < 8 && quarter + 4 * sl < T_) s_st[cg][sl][idx & 3] = r;
  }
  if (a.var) {
    // this chunk's four sums per token of the quarter, the 64-channel groups in order
    __syncthreads();
    const int sl = threadIdx.x >> 2, q = threadIdx.x & 3, i = quarter + 4 * sl;
    if (sl < kMaxTok / 4 && i < T_) {
      const double tot = ((s_st[0][sl][q] + s_st[1][sl][q]) + s_st[2][sl][q]) + s_st[3][sl][q];
      a.stats[((size_t)i * 4 + q) * a.chunks + blockIdx.x] = tot;   // [token][sum][chunk]
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core decode (t >= 2, 16-bit).  With several tokens the union of kept
// channels covers nearly every row of the weight (each token keeps its own
// n of every m), so the product runs as a skinny dense GEMM over the masked
// rows xm that the pruning pass writes in fragment order (zeros at pruned
// channels):
//   y[i][j] = nu_i * sum_k xm[i][k] w[j][k] + eta_i * s_j.
// Workgroup = 64 output rows x a channel range (split), 8 waves.  The weight
// rows and the activation fragments stream through a kMmStages-deep LDS ring
// by direct global->LDS loads (no registers held by loads in flight), one
// stage = kMmSteps 64-channel steps.  Per stage every wave issues the same
// loads: four 1 KB weight loads (two rows x 512 contiguous bytes each; the
// 16-byte chunk c of row r is stored at slot c ^ (r & 15), which makes the
// fragment reads conflict-free) and one 1 KB activation load per 16-token
// block.  So a vmcnt wait means "this stage has landed", and one barrier per
// stage makes it visible and frees the stage refilled next.  Wave w multiplies
// rows 16 (w % 4) .. +15 with window h = w / 4 of each step (mfma 16x16x32;
// lane group g of window h holds channels 16 g + 8 h .. +7, the order of the
// activation fragments); the two windows are added in LDS, then the splits
// through the ticket.  Each workgroup folds nu from the pruning pass's chunk
// sums, loaded ahead of its first stage.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, f32x4 c) {
  if constexpr (DT == SPA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

__device__ __forceinline__ uint4 zero_unless(const uint4& v, bool ok) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

constexpr int kMmStages = 3, kMmRows = 64;   // ring stages of kMmSteps 64-channel steps

template <int TT>
constexpr int mm_stage_bytes() { return kMmRows * 128 * kMmSteps + TT * 2048 * kMmSteps; }

template <int DT, int TT>
__global__ void __launch_bounds__(512) k_decode_mm(DecodeArgs a) {
  using T = typename Dt<DT>::T;
  constexpr int NS = kMmStages, RN = kMmRows, SU = kMmSteps, PER = 4 + TT;
  constexpr int RB = 128 * SU;                             // bytes of one weight row per stage
  constexpr int SW = RN * RB, SS = mm_stage_bytes<TT>();
  static_assert(RN * RB / 1024 == 4 * 8, "four 1 KB weight loads per wave");
  __shared__ __attribute__((aligned(16))) unsigned char s_ring[NS * SS];
  __shared__ float s_nu[kMaxTok];
  __shared__ int s_flag;
  const int T_ = a.t, K = a.k, N = a.n_out;
  const int tile = blockIdx.x % a.tiles, split = blockIdx.x / a.tiles;
  const int n0 = tile * RN;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int rf = wv & 3, hw = wv >> 2;                     // row fragment, window
  const int ntb = (T_ + 15) / 16;

  // this workgroup's 64-channel steps, taken SU at a time ("stages"); each
  // tile starts its walk at a different stage (rows of w lie k*2 bytes apart,
  // so workgroups walking k in step would all hit the same few memory
  // channels at once)
  const int nsteps = (K + 63) / 64;
  const int sps = a.k_len / 64;
  const int s_beg = split * sps, s_end = min(nsteps, s_beg + sps);
  const int span = s_end - s_beg;
  const int nst = (span + SU - 1) / SU;
  const int rot = nst > 0 ? (int)(((unsigned)tile * 37u) % (unsigned)nst) : 0;
  auto stage_of = [&](int i) {                             // first step of stage i
    const int v = i + rot;
    return s_beg + SU * (v >= nst ? v - nst : v);
  };

  // load sources.  Weight: wave w, load j reads 512 contiguous bytes (4 steps)
  // of tile row dr = 8 w + 2 j + lane / 32; lane position p = lane % 32 of the
  // row's LDS run holds channel chunk p ^ (dr & 15) of the stage, which makes
  // the fragment reads (16 rows, one chunk) conflict-free.  Activations: the
  // stage's SU steps x TT token blocks are one contiguous run of the
  // fragment-order buffer, TT 1 KB loads per wave.
  const int dp = lane & 31;
  const T* wbase = static_cast<const T*>(a.w) + (size_t)n0 * K;
  const uint16_t* xf = static_cast<const uint16_t*>(a.dense);
  const uint32_t ring = lds_addr(s_ring);
  auto issue = [&](int i) {                                // stage i into slot i % NS
    const int st0 = stage_of(i);
    const uint32_t q = ring + (uint32_t)(i % NS) * SS;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dr = 8 * wv + 2 * j + (lane >> 5);
      const uint32_t rbytes = (uint32_t)(min(n0 + dr, N - 1) - n0) * (uint32_t)K * 2u;
      const int kc = st0 * 64 + 8 * (dp ^ (dr & 15));       // chunks past k read chunk 0 (their activations are zero)
      lds_dma16_nt(wbase, rbytes + (uint32_t)(kc < K ? kc : 0) * 2u, q + (uint32_t)(wv * 4 + j) * 1024u);
    }
    // steps past this split or past k: any in-bounds activations (multiplied as zeros)
    const int stx = min(st0, nsteps - SU > 0 ? nsteps - SU : 0);
#pragma unroll
    for (int tb = 0; tb < TT; ++tb)
      lds_dma16(xf, (uint32_t)(frag_offset(stx, 0, ntb, 0, 0) * 2) + (uint32_t)(wv * TT + tb) * 1024u + (uint32_t)lane * 16u,
                q + SW + (uint32_t)(wv * TT + tb) * 1024u);
  };

  f32x4 acc[TT];
#pragma unroll
  for (int tb = 0; tb < TT; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool tok_ok[TT];
#pragma unroll
  for (int tb = 0; tb < TT; ++tb) tok_ok[tb] = 16 * tb + l16 < T_;
  const int wr = 16 * rf + l16;                            // this lane's fragment row
  // window h of lane group g is channels 16 g + 8 h .. +7 of a step (the
  // activation fragments' order): weight chunk 8 j + 2 g + h of step j
  const uint32_t xfrag = (uint32_t)SW + (uint32_t)hw * 1024u + (uint32_t)lane * 16u;

  // nu of tokens w, w+8, w+16, w+24 (wave w) from the pruning pass's chunk
  // sums [token][sum][chunk]: lane l takes (token w + 8 (l / 16), sum
  // (l / 4) % 4) and chunks l % 4, l % 4 + 4, ...  Its loads go out before the
  // first stage's (the stage waits then cover them) and are added after the
  // main loop; a fixed two-step butterfly joins the four parts, the same in
  // every workgroup.
  const int npr = lane >> 2, npart = lane & 3;
  const int nti = wv + 8 * (npr >> 2), nq = npr & 3;
  double nld[16];
  const bool nu_one_pass = a.chunks <= 64;
  if (a.var && nu_one_pass) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int c = npart + 4 * u;
      const bool ok = nti < T_ && c < a.chunks;
      nld[u] = a.stats[((size_t)(ok ? nti : 0) * 4 + nq) * a.chunks + (ok ? c : 0)];
    }
  }
  for (int i = 0; i < NS - 1; ++i)
    if (i < nst) issue(i);
  for (int i = 0; i < nst; ++i) {
    if (i + NS - 2 < nst) wait_vm<(NS - 2) * PER>(1);     // the newer stages may still be in flight
    else wait_vm<0>(0);                                    // the last stages: everything issued has landed
    bare_barrier();
    if (i + NS - 1 < nst) issue(i + NS - 1);
    const unsigned char* stg = s_ring + (size_t)(i % NS) * SS;
    const int st0 = stage_of(i);
    const int stx = min(st0, nsteps - SU > 0 ? nsteps - SU : 0);
#pragma unroll
    for (int j = 0; j < SU; ++j) {
      const int st = st0 + j;
      const bool kin = st < s_end && st * 64 + 16 * g + 8 * hw < K;
      const uint4 wfr = *reinterpret_cast<const uint4*>(stg + wr * RB + (((8 * j + 2 * g + hw) ^ (wr & 15)) * 16));
#pragma unroll
      for (int tb = 0; tb < TT; ++tb) {
        // the activation run starts at step stx: step st sits (st - stx) steps in
        const int jx = st - stx;
        const bool in = kin && jx >= 0 && jx < SU;
        const uint4 xv = *reinterpret_cast<const uint4*>(stg + xfrag + ((in ? jx : 0) * TT + tb) * 2048);
        acc[tb] = mfma16<DT>(wfr, zero_unless(xv, in && tok_ok[tb]), acc[tb]);
      }
    }
  }
  if (a.var) {
    double sacc = 0.0;
    if (nu_one_pass) {
#pragma unroll
      for (int u = 0; u < 16; ++u) sacc += (nti < T_ && npart + 4 * u < a.chunks) ? nld[u] : 0.0;
    } else {
      for (int c = npart; c < a.chunks; c += 4)
        if (nti < T_) sacc += a.stats[((size_t)nti * 4 + nq) * a.chunks + c];
    }
    sacc += __shfl_xor(sacc, 1, kWave);
    sacc += __shfl_xor(sacc, 2, kWave);
    double sums[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) sums[qq] = __shfl(sacc, ((lane & 3) * 4 + qq) * 4, kWave);   // lane l < 4: token slot l
    if (lane < 4) {
      const int it = wv + 8 * lane;
      if (it < T_) {
        const float nu = nu_from_stats(sums, a, it, blockIdx.x == 0);
        s_nu[it] = nu;
        if (blockIdx.x == 0 && a.nu_out) a.nu_out[it] = nu;
      }
    }
  } else if ((int)threadIdx.x < T_) {
    s_nu[threadIdx.x] = 1.f;
    if (blockIdx.x == 0 && a.nu_out) a.nu_out[threadIdx.x] = 1.f;
  }
  // D register r of lane (l16, g): output row 16 rf + 4g + r, token 16 tb + l16;
  // the two windows meet in LDS (the ring is free once every wave is past it)
  __syncthreads();
  float (*s_red)[4][TT][16][17] = reinterpret_cast<float (*)[4][TT][16][17]>(s_ring);
#pragma unroll
  for (int tb = 0; tb < TT; ++tb)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_red[hw][rf][tb][4 * g + r][l16] = acc[tb][r];
  __syncthreads();
  auto wg_sum = [&](int j, int tok) {                      // window 0, then window 1
    return s_red[0][j / 16][tok / 16][j % 16][tok % 16] + s_red[1][j / 16][tok / 16][j % 16][tok % 16];
  };
  const int rows = min(RN, N - n0);
  if (a.splits > 1) {
    for (int e = threadIdx.x; e < rows * T_; e += 512) {
      const int tok = e / rows, j = e % rows;
      coherent_store(&a.partial[((size_t)split * T_ + tok) * N + n0 + j], wg_sum(j, tok));
    }
    if (!arrive_last(&a.counters[tile], a.splits, &s_flag)) return;
  }
  // Final sums of this tile (the last workgroup when split).
  // this thread's (row, token) pairs e = thread + 512 q; with splits, every
  // pair's partials of a batch of 8 splits are in flight before the adds
  // (split order)
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.splits > 1) {
    const size_t stride = (size_t)T_ * N;
    for (int s0 = 0; s0 < a.splits; s0 += 8) {
      float part[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = threadIdx.x + 512 * q;
        const bool ok = e < rows * T_;
        const float* pp = a.partial + (size_t)(ok ? e / rows : 0) * N + n0 + (ok ? e % rows : 0);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
          part[q][s2] = ok && s0 + s2 < a.splits ? coherent_load(pp + (s0 + s2) * stride) : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
          if (s0 + s2 < a.splits) v[q] += part[q][s2];
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = threadIdx.x + 512 * q;
      if (e < rows * T_) v[q] = wg_sum(e % rows, e / rows);
    }
  }
  __syncthreads();
  T* y = static_cast<T*>(a.y);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x + 512 * q;
    if (e < rows * T_) {
      const int tok = e / rows, j = e % rows, col = n0 + j;
      float out = s_nu[tok] * v[q];
      if (a.shift != SPA_SHIFT_NONE) out += a.eta[tok] * a.row_sum[col];
      y[(size_t)tok * N + col] = from_f32<DT>(out);
    }
  }
}

// ---------------------------------------------------------------------------
// Host planning and launch
// ---------------------------------------------------------------------------
size_t decode_workspace(int t, int k, int n_out, int dtype, int n, int m, int score, int shift, int var,
                        DecodeArgs* plan) {
  const DecodePlan p = plan_decode(t, k, n_out, dtype, n, m, var);
  if (plan) {
    DecodeArgs a{};
    a.t = t; a.k = k; a.n_out = n_out; a.n = n; a.m = m; a.score = score; a.shift = shift; a.var = var;
    a.tiles = p.tiles; a.splits = p.splits; a.k_len = p.k_len; a.col_tile = p.col_tile;
    a.chunks = p.chunks; a.list_cap = p.list_cap; a.chunk_blocks = p.chunk_blocks;
    // offsets into the workspace; the caller adds its base address
    a.partial = reinterpret_cast<float*>(p.partial);
    a.stats = reinterpret_cast<double*>(p.stats);
    a.counters = reinterpret_cast<unsigned*>(p.counters);
    a.eta_ws = reinterpret_cast<float*>(p.eta);
    a.dense = reinterpret_cast<void*>(p.dense);
    *plan = a;
  }
  return p.bytes;
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
  if constexpr (DT != SPA_F32) {
    if (t1_kernel(a.t, DT, a.k, a.n_out)) {
      if (a.act)
        hipLaunchKernelGGL((k_decode_t1<DT, M, true>), dim3(a.tiles * a.splits), dim3(kT1Threads), 0, st, a);
      else
        hipLaunchKernelGGL((k_decode_t1<DT, M, false>), dim3(a.tiles * a.splits), dim3(kT1Threads), 0, st, a);
      return hipGetLastError();
    }
  }
  if (a.t <= 1) return fused_launch<DT, M, 1>(a, st);
  if constexpr (DT == SPA_F32) {                    // 16-bit t >= 2 takes the matrix-core path
    if (a.t <= 2) return fused_launch<DT, M, 2>(a, st);
    if (a.t <= 4) return fused_launch<DT, M, 4>(a, st);
    return fused_launch<DT, M, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

template <int DT>
static hipError_t decode_dt(DecodeArgs& a, hipStream_t st) {
  const bool fused = !decode_on_matrix_cores(a.t, DT);
  // the token mean ahead of the main kernel for long rows; shorter calls form
  // it inside the fused kernel or the matrix-core path's pruning pass
  const bool mean_first = (size_t)a.t * a.k > 65536;
  if (a.shift == SPA_SHIFT_TOKEN_MEAN && mean_first) {
    if (hipError_t e = launch_token_mean(DT, a.x, a.t, a.k, a.act, a.eta_ws, st)) return e;
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
    // prune every token once (score, top-n, masked rows, positions, variance sums) ...
    const dim3 pg(a.chunks, 4);                     // channel chunks x token quarters
    switch (a.m) {
      case 4: hipLaunchKernelGGL((k_prune_cols<DT, 4>), pg, dim3(kPcThreads), 0, st, a); break;
      case 8: hipLaunchKernelGGL((k_prune_cols<DT, 8>), pg, dim3(kPcThreads), 0, st, a); break;
      case 16: hipLaunchKernelGGL((k_prune_cols<DT, 16>), pg, dim3(kPcThreads), 0, st, a); break;
      default: hipLaunchKernelGGL((k_prune_cols<DT, 32>), pg, dim3(kPcThreads), 0, st, a); break;
    }
    if (hipError_t e = hipGetLastError()) return e;
    if (a.shift == SPA_SHIFT_TOKEN_MEAN) a.eta = a.eta_ws;   // the means the pass (or the mean pass) wrote
    // ... then one pass over the row-major weight on the matrix cores
    if (a.t <= 16)
      hipLaunchKernelGGL((k_decode_mm<DT, 1>), dim3(a.tiles * a.splits), dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((k_decode_mm<DT, 2>), dim3(a.tiles * a.splits), dim3(512), 0, st, a);
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

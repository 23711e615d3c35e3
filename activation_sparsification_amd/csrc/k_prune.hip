// Pruning pass: shift, score, per-block top-n, pack, variance factor.
//
// One workgroup (256 threads) per token row.  Each lane owns a segment of
// max(16, m) consecutive channels -- whole m-blocks -- and ranks every block
// in registers (guide s2.1: keep n of every m; ties to the lower channel
// index, so exactly n survive): six pairwise comparisons for m = 4, the
// selection network of spa_select.h for wider blocks.
//
// Outputs (any subset): packed values + uint8 in-block positions; the
// 2:4 nibble metadata the sparse MFMA consumes; or masked dense rows for
// the dense-MFMA path of other n:m patterns.
#include "spa_common.h"
#include "spa_launch.h"
#include "spa_select.h"

namespace spa {

// One segment of a row as raw 16-byte words through a buffer descriptor over
// the row (an offset past the row reads zeros, so the load needs no branch).
template <int DT, int SEG>
struct RawSeg {
  static constexpr int NQ = SEG * Dt<DT>::bytes / 16;
  uint4 q[NQ];
};
template <int DT, int SEG>
__device__ __forceinline__ void load_raw(__amdgpu_buffer_rsrc_t r, int seg, bool ok, RawSeg<DT, SEG>& out) {
#pragma unroll
  for (int i = 0; i < RawSeg<DT, SEG>::NQ; ++i)
    out.q[i] = buffer_load16(r, ok ? (uint32_t)(seg * SEG * Dt<DT>::bytes + 16 * i) : kBufferOutOfRange);
}
template <int DT, int SEG>
__device__ __forceinline__ void unpack_raw(const RawSeg<DT, SEG>& in, int act, float (&v)[SEG]) {
  if constexpr (DT == SPA_F32) {
#pragma unroll
    for (int i = 0; i < SEG / 4; ++i) {
      v[4 * i] = __uint_as_float(in.q[i].x); v[4 * i + 1] = __uint_as_float(in.q[i].y);
      v[4 * i + 2] = __uint_as_float(in.q[i].z); v[4 * i + 3] = __uint_as_float(in.q[i].w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < SEG / 8; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[8 * i + e] = elem16<DT>(in.q[i], e);
  }
  if (act) {
#pragma unroll
    for (int j = 0; j < SEG; ++j) v[j] = relu2<DT>(v[j]);
  }
}

// Keep bits of one m-block (bit j set = channel j kept).
template <int M>
__device__ __forceinline__ uint32_t block_keep(const float* sc, int n) {
  int rank[M];
#pragma unroll
  for (int j = 0; j < M; ++j) rank[j] = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
#pragma unroll
    for (int q = j + 1; q < M; ++q) {
      // j < q: j beats q unless q's score is strictly larger.
      const bool jwins = sc[j] >= sc[q];
      rank[q] += jwins ? 1 : 0;
      rank[j] += jwins ? 0 : 1;
    }
  }
  uint32_t keep = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) keep |= (rank[j] < n ? 1u : 0u) << j;
  return keep;
}

// Token mean of a long row: 16-byte loads, four in flight per thread, four
// float64 partial sums combined in a fixed order, then the workgroup sum.
template <int DT>
__device__ __forceinline__ float row_mean(const typename Dt<DT>::T* __restrict__ row, int k, int act, double* s_red) {
  constexpr int PER = 16 / Dt<DT>::bytes;
  const int nq = k / PER;
  double part[4] = {0.0, 0.0, 0.0, 0.0};
  for (int q0 = 0; q0 < nq; q0 += 4 * 256) {
    uint4 u[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = q0 + r * 256 + (int)threadIdx.x;
      u[r] = q < nq ? reinterpret_cast<const uint4*>(row)[q] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (DT == SPA_F32) {
        part[r] += ((double)apply_act<DT>(__uint_as_float(u[r].x), act) +
                    (double)apply_act<DT>(__uint_as_float(u[r].y), act)) +
                   ((double)apply_act<DT>(__uint_as_float(u[r].z), act) +
                    (double)apply_act<DT>(__uint_as_float(u[r].w), act));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) part[r] += (double)apply_act<DT>(elem16<DT>(u[r], e), act);
      }
    }
  }
  const double tot = block_sum((part[0] + part[1]) + (part[2] + part[3]), s_red);
  return (float)(tot / (double)k);
}

template <int DT, int M>
__global__ void __launch_bounds__(256) k_prune(PruneArgs a) {
  using T = typename Dt<DT>::T;
  constexpr int SEG = M > 16 ? M : 16;
  constexpr int BPS = SEG / M;
  __shared__ double s_red[4];
  // staging for packed outputs of one wave-iteration: 64 lanes x SEG*n/m values
  extern __shared__ unsigned char s_dyn[];

  const int row = blockIdx.x;
  const int n = a.n;
  const int kept_row = a.k / M * n;        // packed values per row
  const int kept_seg = BPS * n;            // packed values per segment
  const T* xr = static_cast<const T*>(a.x) + (size_t)row * a.k;

  const int nseg = a.k / SEG;
  // All lanes of a wave run the same number of iterations so the wave-wide
  // copy-out below stays convergent.
  const int iters = (nseg + 255) / 256;
  // the first pass's segment is requested before the shift is known; when the
  // whole row is one pass, the shift is summed from these same registers.
  // Each pass then requests the next pass's segment before its own work.
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(xr), (short)0, a.k * (int)sizeof(T), kBufferWord3);
  RawSeg<DT, SEG> raw_next;
  load_raw<DT, SEG>(xrs, (int)threadIdx.x, (int)threadIdx.x < nseg, raw_next);
  float xv0[SEG];
  unpack_raw<DT, SEG>(raw_next, a.act, xv0);
  float eta = 0.f;
  if (a.shift_mean) {
    if (iters == 1) {
      double s = 0.0;
      if ((int)threadIdx.x < nseg) {
#pragma unroll
        for (int j = 0; j < SEG; ++j) s += (double)xv0[j];
      }
      eta = (float)(block_sum(s, s_red) / (double)a.k);
    } else {
      eta = row_mean<DT>(xr, a.k, a.act, s_red);
    }
  } else if (a.eta_given) {
    eta = a.eta_given[row];
  }
  if (threadIdx.x == 0) {
    if (a.eta_out) a.eta_out[row] = eta;
  }
  // FP8 packing: the token's scale from max |x - eta| over the row (the
  // registers of the one-pass case, else a second read of the row)
  float fp8_inv = 0.f;
  if (a.fp8) {
    float mx = 0.f;
    if (iters == 1) {
      if ((int)threadIdx.x < nseg) {
#pragma unroll
        for (int j = 0; j < SEG; ++j) mx = fmaxf(mx, __builtin_fabsf(xv0[j] - eta));
      }
    } else {
      for (int sg = threadIdx.x; sg < nseg; sg += 256) {
        RawSeg<DT, SEG> r2;
        load_raw<DT, SEG>(xrs, sg, true, r2);
        float v2[SEG];
        unpack_raw<DT, SEG>(r2, a.act, v2);
#pragma unroll
        for (int j = 0; j < SEG; ++j) mx = fmaxf(mx, __builtin_fabsf(v2[j] - eta));
      }
    }
    __shared__ float s_mx[4];
    const float amax = block_max(mx, s_mx);
    float scale;
    fp8_scales(amax, scale, fp8_inv);
    if (threadIdx.x == 0) a.fp8_scale[row] = scale;
  }

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  T* s_vals = reinterpret_cast<T*>(s_dyn) + (size_t)wv * 64 * kept_seg;
  uint8_t* s_idx = reinterpret_cast<uint8_t*>(s_dyn + (size_t)4 * 64 * kept_seg * sizeof(T)) + (size_t)wv * 64 * kept_seg;

  double sx = 0.0, sxx = 0.0, sm = 0.0, smm = 0.0;
  for (int it = 0; it < iters; ++it) {
    const int seg = it * 256 + threadIdx.x;
    const bool active = seg < nseg;
    uint32_t keepbits[BPS];
    float xh[SEG];
    float xv[SEG];
    if (it == 0) {
#pragma unroll
      for (int j = 0; j < SEG; ++j) xv[j] = xv0[j];
    } else {
      unpack_raw<DT, SEG>(raw_next, a.act, xv);
    }
    if (it + 1 < iters) load_raw<DT, SEG>(xrs, seg + 256, seg + 256 < nseg, raw_next);
    if (active) {
#pragma unroll
      for (int j = 0; j < SEG; ++j) xh[j] = xv[j] - eta;
      float sc[SEG];
      if (a.colnorm) {
        const float* f = a.colnorm + (size_t)seg * SEG;
#pragma unroll
        for (int j = 0; j < SEG; ++j) sc[j] = __builtin_fabsf(xh[j]) * f[j];
      } else if (a.chan_scale) {
        const float* f = a.chan_scale + (size_t)seg * SEG;
#pragma unroll
        for (int j = 0; j < SEG; ++j) sc[j] = __builtin_fabsf(xh[j]) * f[j];
      } else {
#pragma unroll
        for (int j = 0; j < SEG; ++j) sc[j] = __builtin_fabsf(xh[j]);
      }
#pragma unroll
      for (int b = 0; b < BPS; ++b) {
        if constexpr (M >= 8) {            // selection network on the score bits
          uint32_t sb[M];
#pragma unroll
          for (int j = 0; j < M; ++j) sb[j] = __float_as_uint(sc[b * M + j]);
          keepbits[b] = topn_keep_bits<M>(sb, n);
        } else {                           // 4 channels: six pairwise comparisons
          keepbits[b] = block_keep<M>(sc + b * M, n);
        }
      }

      if (a.var) {
#pragma unroll
        for (int b = 0; b < BPS; ++b)
#pragma unroll
          for (int j = 0; j < M; ++j) {
            const double v = (double)xh[b * M + j];
            sx += v;
            sxx += v * v;
            if ((keepbits[b] >> j) & 1u) { sm += v; smm += v * v; }
          }
      }
      if (a.pack & kPackTiled24) {
        // 2:4: the segment's 16 channels are 4 blocks -> 8 kept values (16 bytes) and
        // one 16-bit word of positions, stored at step seg / 4, slot seg % 4
        if constexpr (M == 4 && DT != SPA_F32) {
          uint32_t meta = 0;
          uint32_t wds[4];
          float flo[4], fhi[4];
#pragma unroll
          for (int b = 0; b < BPS; ++b) {
            const uint32_t kb = keepbits[b];
            const uint32_t lo = __builtin_ctz(kb);
            const uint32_t hi = 31 - __builtin_clz(kb);
            meta |= (lo | (hi << 2)) << (4 * b);
            float vlo = xh[4 * b], vhi = xh[4 * b];
#pragma unroll
            for (int j = 1; j < 4; ++j) {
              vlo = (int)lo == j ? xh[4 * b + j] : vlo;
              vhi = (int)hi == j ? xh[4 * b + j] : vhi;
            }
            flo[b] = vlo;
            fhi[b] = vhi;
            wds[b] = (uint32_t)from_f32<DT>(vlo) | ((uint32_t)from_f32<DT>(vhi) << 16);
          }
          const size_t rowpos = (size_t)(seg / 4) * a.t_pad + row;
          if (a.fp8) {
            // the eight kept values as e4m3 codes of x_hat * (448 / max), in
            // channel order: 8 bytes at slot seg % 4 of the row's 32 bytes
            const uint32_t q01 = fp8_pair(flo[0] * fp8_inv, fhi[0] * fp8_inv) |
                                 (fp8_pair(flo[1] * fp8_inv, fhi[1] * fp8_inv) << 16);
            const uint32_t q23 = fp8_pair(flo[2] * fp8_inv, fhi[2] * fp8_inv) |
                                 (fp8_pair(flo[3] * fp8_inv, fhi[3] * fp8_inv) << 16);
            reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.tiled_vals) + rowpos * 32)[seg % 4] = make_uint2(q01, q23);
          } else {
            reinterpret_cast<uint4*>(static_cast<T*>(a.tiled_vals) + rowpos * 32)[seg % 4] =
                make_uint4(wds[0], wds[1], wds[2], wds[3]);
          }
          a.tiled_meta[rowpos * 4 + seg % 4] = (uint16_t)meta;
        }
      }
      if (a.pack & kPackDense) {
        T* d = static_cast<T*>(a.dense) + (size_t)row * a.k + (size_t)seg * SEG;
        if constexpr (DT == SPA_F32) {
#pragma unroll
          for (int i = 0; i < SEG / 4; ++i) {
            float4 f;
            f.x = ((keepbits[(4 * i) / M] >> ((4 * i) % M)) & 1u) ? xh[4 * i] : 0.f;
            f.y = ((keepbits[(4 * i + 1) / M] >> ((4 * i + 1) % M)) & 1u) ? xh[4 * i + 1] : 0.f;
            f.z = ((keepbits[(4 * i + 2) / M] >> ((4 * i + 2) % M)) & 1u) ? xh[4 * i + 2] : 0.f;
            f.w = ((keepbits[(4 * i + 3) / M] >> ((4 * i + 3) % M)) & 1u) ? xh[4 * i + 3] : 0.f;
            reinterpret_cast<float4*>(d)[i] = f;
          }
        } else {
#pragma unroll
          for (int i = 0; i < SEG / 8; ++i) {
            uint32_t wds[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const int j0 = 8 * i + 2 * p, j1 = j0 + 1;
              const uint32_t v0 = ((keepbits[j0 / M] >> (j0 % M)) & 1u) ? (uint32_t)from_f32<DT>(xh[j0]) : 0u;
              const uint32_t v1 = ((keepbits[j1 / M] >> (j1 % M)) & 1u) ? (uint32_t)from_f32<DT>(xh[j1]) : 0u;
              wds[p] = v0 | (v1 << 16);
            }
            reinterpret_cast<uint4*>(d)[i] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
          }
        }
      }
      if (a.pack & kPackVals) {
        // Kept values in ascending channel order, staged per wave in LDS.
        int pos = lane * kept_seg;
#pragma unroll
        for (int j = 0; j < SEG; ++j) {
          if ((keepbits[j / M] >> (j % M)) & 1u) {
            s_vals[pos] = from_f32<DT>(xh[j]);
            s_idx[pos] = (uint8_t)(j % M);
            ++pos;
          }
        }
      }
    }
    if (a.pack & kPackVals) {
      // Copy the wave's contiguous run of packed values out.
      __syncthreads();
      const int seg0 = it * 256 + wv * 64;
      const int nseg_w = min(64, nseg - seg0);
      if (nseg_w > 0) {
        const int cnt = nseg_w * kept_seg;
        T* vdst = a.vals ? static_cast<T*>(a.vals) + (size_t)row * kept_row + (size_t)seg0 * kept_seg : nullptr;
        if (a.vals)
          for (int e = lane; e < cnt; e += 64) vdst[e] = s_vals[e];
        if (a.idx) {
          uint8_t* idst = a.idx + (size_t)row * kept_row + (size_t)seg0 * kept_seg;
          for (int e = lane; e < cnt; e += 64) idst[e] = s_idx[e];
        }
      }
      __syncthreads();
    }
  }

  if (a.var || a.nu_out) {
    float nu = 1.f;
    if (a.var) {
      const double tx = block_sum(sx, s_red);
      const double txx = block_sum(sxx, s_red);
      const double tm = block_sum(sm, s_red);
      const double tmm = block_sum(smm, s_red);
      const double kk = (double)a.k;
      const double var_full = txx / kk - (tx / kk) * (tx / kk);
      const double var_mask = tmm / kk - (tm / kk) * (tm / kk);
      nu = nu_of(var_full, var_mask, a.var, a.var_in, a.var_out, row, threadIdx.x == 0);
    }
    if (threadIdx.x == 0 && a.nu_out) a.nu_out[row] = nu;
  }
}

template <int DT>
__global__ void __launch_bounds__(256) k_token_mean(const typename Dt<DT>::T* __restrict__ x, int k, int act,
                                                    float* __restrict__ eta) {
  __shared__ double s_red[4];
  const float e = row_mean<DT>(x + (size_t)blockIdx.x * k, k, act, s_red);
  if (threadIdx.x == 0) eta[blockIdx.x] = e;
}

// Static shift table (the guide's s3.1, S-PTS): calibration adds each token's
// dynamic shift (the same float32 token mean as above) and a count under the
// token's id; the table entry is their mean.  The float64 additions are
// atomic, so their order (and the last bits of a sum) may vary between runs.
template <int DT>
__global__ void __launch_bounds__(256) k_eta_accum(const typename Dt<DT>::T* __restrict__ x, int k,
                                                   const int32_t* __restrict__ ids, int vocab, double* sums,
                                                   uint32_t* counts) {
  __shared__ double s_red[4];
  const float e = row_mean<DT>(x + (size_t)blockIdx.x * k, k, 0, s_red);
  if (threadIdx.x == 0) {
    const int id = ids[blockIdx.x];
    if (id >= 0 && id < vocab) {
      atomicAdd(&sums[id], (double)e);
      atomicAdd(&counts[id], 1u);
    }
  }
}

__global__ void __launch_bounds__(256) k_eta_finalize(const double* __restrict__ sums,
                                                      const uint32_t* __restrict__ counts, int vocab,
                                                      float* __restrict__ table) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < vocab) table[i] = counts[i] ? (float)(sums[i] / (double)counts[i]) : 0.f;
}

__global__ void __launch_bounds__(256) k_eta_lookup(const float* __restrict__ table, int vocab,
                                                    const int32_t* __restrict__ ids, int t, float* __restrict__ eta) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < t) {
    const int id = ids[i];
    eta[i] = (id >= 0 && id < vocab) ? table[id] : 0.f;
  }
}

hipError_t launch_eta_calibrate(int dtype, const void* x, int t, int k, const int32_t* ids, int vocab, double* sums,
                                uint32_t* counts, hipStream_t st) {
  if (t == 0) return hipSuccess;
  switch (dtype) {
    case SPA_F32:
      hipLaunchKernelGGL(k_eta_accum<SPA_F32>, dim3(t), dim3(256), 0, st, (const float*)x, k, ids, vocab, sums,
                         counts);
      break;
    case SPA_F16:
      hipLaunchKernelGGL(k_eta_accum<SPA_F16>, dim3(t), dim3(256), 0, st, (const uint16_t*)x, k, ids, vocab, sums,
                         counts);
      break;
    default:
      hipLaunchKernelGGL(k_eta_accum<SPA_BF16>, dim3(t), dim3(256), 0, st, (const uint16_t*)x, k, ids, vocab, sums,
                         counts);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_eta_table(const double* sums, const uint32_t* counts, int vocab, float* table, hipStream_t st) {
  if (vocab == 0) return hipSuccess;
  hipLaunchKernelGGL(k_eta_finalize, dim3((vocab + 255) / 256), dim3(256), 0, st, sums, counts, vocab, table);
  return hipGetLastError();
}

hipError_t launch_eta_lookup(const float* table, int vocab, const int32_t* ids, int t, float* eta, hipStream_t st) {
  if (t == 0) return hipSuccess;
  hipLaunchKernelGGL(k_eta_lookup, dim3((t + 255) / 256), dim3(256), 0, st, table, vocab, ids, t, eta);
  return hipGetLastError();
}

// CLACT column energy, one thread per channel, tokens in ascending order.
template <int DT>
__global__ void __launch_bounds__(256) k_colnorm(const typename Dt<DT>::T* __restrict__ x, int act,
                                                 const float* __restrict__ eta, int t, int k, float* __restrict__ c) {
  const int ch = blockIdx.x * 256 + threadIdx.x;
  if (ch >= k) return;
  float acc = 0.f;
  for (int p = 0; p < t; ++p) {
    const float v = apply_act<DT>(to_f32<DT>(x[(size_t)p * k + ch]), act) - (eta ? eta[p] : 0.f);
    acc = clact_accumulate(acc, v);
  }
  c[ch] = sqrt_rn(acc);
}

template <int DT, int M>
static hipError_t prune_m(const PruneArgs& a, hipStream_t st) {
  constexpr int SEG = M > 16 ? M : 16;
  const int kept_seg = SEG / M * a.n;
  const size_t lds = (a.pack & kPackVals) ? (size_t)4 * 64 * kept_seg * (Dt<DT>::bytes + 1) : 0;
  hipLaunchKernelGGL((k_prune<DT, M>), dim3(a.t), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <int DT>
static hipError_t prune_dt(const PruneArgs& a, hipStream_t st) {
  switch (a.m) {
    case 4: return prune_m<DT, 4>(a, st);
    case 8: return prune_m<DT, 8>(a, st);
    case 16: return prune_m<DT, 16>(a, st);
    default: return prune_m<DT, 32>(a, st);
  }
}

hipError_t launch_prune(int dtype, const PruneArgs& a, hipStream_t st) {
  if (a.t == 0) return hipSuccess;
  switch (dtype) {
    case SPA_F32: return prune_dt<SPA_F32>(a, st);
    case SPA_F16: return prune_dt<SPA_F16>(a, st);
    default: return prune_dt<SPA_BF16>(a, st);
  }
}

hipError_t launch_token_mean(int dtype, const void* x, int t, int k, int act, float* eta, hipStream_t st) {
  if (t == 0) return hipSuccess;
  switch (dtype) {
    case SPA_F32:
      hipLaunchKernelGGL(k_token_mean<SPA_F32>, dim3(t), dim3(256), 0, st, (const float*)x, k, act, eta);
      break;
    case SPA_F16:
      hipLaunchKernelGGL(k_token_mean<SPA_F16>, dim3(t), dim3(256), 0, st, (const uint16_t*)x, k, act, eta);
      break;
    default:
      hipLaunchKernelGGL(k_token_mean<SPA_BF16>, dim3(t), dim3(256), 0, st, (const uint16_t*)x, k, act, eta);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_colnorm(int dtype, const void* x, int act, const float* eta, int t, int k, float* c,
                          hipStream_t st) {
  const dim3 grid((k + 255) / 256);
  switch (dtype) {
    case SPA_F32:
      hipLaunchKernelGGL(k_colnorm<SPA_F32>, grid, dim3(256), 0, st, (const float*)x, act, eta, t, k, c);
      break;
    case SPA_F16:
      hipLaunchKernelGGL(k_colnorm<SPA_F16>, grid, dim3(256), 0, st, (const uint16_t*)x, act, eta, t, k, c);
      break;
    default:
      hipLaunchKernelGGL(k_colnorm<SPA_BF16>, grid, dim3(256), 0, st, (const uint16_t*)x, act, eta, t, k, c);
      break;
  }
  return hipGetLastError();
}

}  // namespace spa

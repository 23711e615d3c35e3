// Pruning pass: shift, score, per-block top-n, pack, variance factor.
//
// k_prune: one workgroup (256 threads) per token row.  Each lane owns a
// segment of max(16, m) consecutive channels -- whole m-blocks -- and ranks
// every block in registers (guide s2.1: keep n of every m; ties to the lower
// channel index, so exactly n survive): for 2:4 the four-comparison
// tournament of spa_select.h, six pairwise comparisons for other n of 4, the
// selection network of spa_select.h for wider blocks.
//
// Outputs (any subset): packed values + uint8 in-block positions; the
// 2:4 nibble metadata the sparse MFMA consumes; or masked dense rows for
// the dense-MFMA path of other n:m patterns.  Calls that want only the 2:4
// operand of 16-bit rows take the lean passes further down (k_prune24,
// k_prune24_rows).
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

// Keep bits of the BPS = SEG / M blocks of one segment of shifted values:
// score |x_hat| times the CLACT column norm or the weight factor (or alone),
// then the top n of every m-block.
template <int M, int SEG>
__device__ __forceinline__ void seg_keep(const float (&xh)[SEG], int seg, const PruneArgs& a, uint32_t (&keep)[SEG / M]) {
  float sc[SEG];
  const float* f = a.colnorm ? a.colnorm + (size_t)seg * SEG : a.chan_scale ? a.chan_scale + (size_t)seg * SEG : nullptr;
  if (f) {
#pragma unroll
    for (int j = 0; j < SEG; ++j) sc[j] = __builtin_fabsf(xh[j]) * f[j];
  } else {
#pragma unroll
    for (int j = 0; j < SEG; ++j) sc[j] = __builtin_fabsf(xh[j]);
  }
#pragma unroll
  for (int b = 0; b < SEG / M; ++b) {
    if constexpr (M >= 8) {            // selection network on the score bits
      uint32_t sb[M];
#pragma unroll
      for (int j = 0; j < M; ++j) sb[j] = __float_as_uint(sc[b * M + j]);
      keep[b] = topn_keep_bits<M>(sb, a.n);
    } else {                           // 4 channels: six pairwise comparisons
      keep[b] = block_keep<M>(sc + b * M, a.n);
    }
  }
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

// Running max of |x - eta| over the kept entries of one segment (the FP8
// token scale is taken over the sparsified row).
template <int M, int SEG>
__device__ __forceinline__ float kept_absmax(const float (&v)[SEG], float eta, int seg, const PruneArgs& a, float mx) {
  float xh[SEG];
#pragma unroll
  for (int j = 0; j < SEG; ++j) xh[j] = v[j] - eta;
  if constexpr (M == 4) {
    if (a.n == 2) {
      const float* f = a.colnorm ? a.colnorm + (size_t)seg * SEG : a.chan_scale ? a.chan_scale + (size_t)seg * SEG : nullptr;
#pragma unroll
      for (int b = 0; b < SEG / 4; ++b) {
        float sc[4], lo, hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j] = f ? __builtin_fabsf(xh[4 * b + j]) * f[4 * b + j] : __builtin_fabsf(xh[4 * b + j]);
        top2of4(sc, xh + 4 * b, lo, hi);
        mx = fmaxf(mx, fmaxf(__builtin_fabsf(lo), __builtin_fabsf(hi)));
      }
      return mx;
    }
  }
  uint32_t kb[SEG / M];
  seg_keep<M, SEG>(xh, seg, a, kb);
#pragma unroll
  for (int j = 0; j < SEG; ++j)
    if ((kb[j / M] >> (j % M)) & 1u) mx = fmaxf(mx, __builtin_fabsf(xh[j]));
  return mx;
}

// Block index -> row such that XCD x (blocks b with b % 8 == x) gets rows
// [x q, x q + q), q = t / 8; the last t % 8 rows keep their own index.
__device__ __forceinline__ int xcd_contiguous(int b, int t) {
  const int q = t / 8;
  return b < 8 * q ? (b % 8) * q + b / 8 : b;
}

template <int DT, int M>
__global__ void __launch_bounds__(256) k_prune(PruneArgs a) {
  using T = typename Dt<DT>::T;
  constexpr int SEG = M > 16 ? M : 16;
  constexpr int BPS = SEG / M;
  __shared__ double s_red[4];
  // staging for packed outputs of one wave-iteration: 64 lanes x SEG*n/m values
  extern __shared__ unsigned char s_dyn[];

  // Workgroup b runs on XCD b % 8; each XCD takes a contiguous run of rows,
  // so the rows that share a line of the step-major packed layout (16 rows of
  // 8-byte position words, 2 rows of 64-byte values) are written through one
  // L2, which merges them into whole lines before they reach memory.
  const int row = xcd_contiguous(blockIdx.x, a.t);
  const int n = a.n;
  const int kept_row = a.k / M * n;        // packed values per row
  const int kept_seg = BPS * n;            // packed values per segment
  const T* xr = static_cast<const T*>(a.x) + (size_t)row * a.k;

  const int nseg = a.k / SEG;
  // All lanes of a wave run the same number of passes so the wave-wide
  // copy-out below stays convergent.
  const int iters = (nseg + 255) / 256;
  // A ring of G segment loads per thread (at most 32 data registers): pass p
  // is requested G passes before its use, so a workgroup keeps G x 256
  // segments of its row outstanding.  A row of at most G passes is read once:
  // the shift and the FP8 scale come from these same registers.
  constexpr int NQ = RawSeg<DT, SEG>::NQ;
  constexpr int G = NQ >= 8 ? 1 : 8 / NQ;
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(xr), (short)0, a.k * (int)sizeof(T), kBufferWord3);
  RawSeg<DT, SEG> raw[G];
#pragma unroll
  for (int u = 0; u < G; ++u) {
    const int sg = u * 256 + (int)threadIdx.x;
    load_raw<DT, SEG>(xrs, sg, sg < nseg, raw[u]);
  }
  const bool resident = iters <= G;
  float eta = 0.f;
  if (a.shift_mean) {
    if (resident) {
      double s = 0.0;
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (u * 256 + (int)threadIdx.x < nseg) {
          float v[SEG];
          unpack_raw<DT, SEG>(raw[u], a.act, v);
#pragma unroll
          for (int j = 0; j < SEG; ++j) s += (double)v[j];
        }
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
  // FP8 packing quantises the sparsified row: the token's scale comes from
  // max |x - eta| over the kept entries (selected here first, from the
  // registers of a resident row, else from a second read of the row)
  float fp8_inv = 0.f;
  if (a.fp8) {
    float mx = 0.f;
    if (resident) {
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int sg = u * 256 + (int)threadIdx.x;
        if (sg < nseg) {
          float v[SEG];
          unpack_raw<DT, SEG>(raw[u], a.act, v);
          mx = kept_absmax<M, SEG>(v, eta, sg, a, mx);
        }
      }
    } else {
      for (int sg = threadIdx.x; sg < nseg; sg += 256) {
        RawSeg<DT, SEG> r2;
        load_raw<DT, SEG>(xrs, sg, true, r2);
        float v[SEG];
        unpack_raw<DT, SEG>(r2, a.act, v);
        mx = kept_absmax<M, SEG>(v, eta, sg, a, mx);
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
  // One pass: this thread's segment `it * 256 + tid` of the row.
  auto pass = [&](int it, const float (&xv)[SEG]) {
    const int seg = it * 256 + threadIdx.x;
    if (seg < nseg) {
      uint32_t keepbits[BPS];
      float xh[SEG];
#pragma unroll
      for (int j = 0; j < SEG; ++j) xh[j] = xv[j] - eta;
      // 2:4 (the only pattern of the tiled operand): each block's position
      // code, four to a 16-bit word, and its two kept values, by tournament;
      // the keep bits only where an output needs them
      uint32_t meta24 = 0;
      float flo[BPS], fhi[BPS];
      if (M == 4 && n == 2) {
        if constexpr (M == 4) {
          const float* f = a.colnorm ? a.colnorm + (size_t)seg * SEG : a.chan_scale ? a.chan_scale + (size_t)seg * SEG : nullptr;
#pragma unroll
          for (int b = 0; b < BPS; ++b) {
            float sc[4];
            if (f) {
#pragma unroll
              for (int j = 0; j < 4; ++j) sc[j] = __builtin_fabsf(xh[4 * b + j]) * f[4 * b + j];
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) sc[j] = __builtin_fabsf(xh[4 * b + j]);
            }
            meta24 |= top2of4(sc, xh + 4 * b, flo[b], fhi[b]) << (4 * b);
          }
          if (a.var || (a.pack & (kPackDense | kPackVals))) {
#pragma unroll
            for (int b = 0; b < BPS; ++b) {
              const uint32_t code = meta24 >> (4 * b);
              keepbits[b] = (1u << (code & 3u)) | (1u << ((code >> 2) & 3u));
            }
          }
        }
      } else {
        seg_keep<M, SEG>(xh, seg, a, keepbits);
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
          uint32_t wds[4];
#pragma unroll
          for (int b = 0; b < BPS; ++b) wds[b] = pack2<DT>(flo[b], fhi[b]);
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
          a.tiled_meta[rowpos * 4 + seg % 4] = (uint16_t)meta24;
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
  };
  for (int g = 0; g < iters; g += G) {
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int it = g + u;
      if (it < iters) {                  // the same for the whole workgroup
        float xv[SEG];
        unpack_raw<DT, SEG>(raw[u], a.act, xv);
        if (it + G < iters) {
          const int nx = (it + G) * 256 + (int)threadIdx.x;
          load_raw<DT, SEG>(xrs, nx, nx < nseg, raw[u]);
        }
        pass(it, xv);
      }
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

// The 2:4 sparse-MFMA operand alone (16-bit rows of at most 16384 channels;
// no variance factor and no separate positions): the same shift, score,
// selection and packing as k_prune, laid out for throughput.
//
// A grid of about a thousand workgroups walks the rows: the j-th row of
// workgroup b is xcd_contiguous(j * grid + b), so at every step the
// workgroups of one XCD hold adjacent rows and their stores meet in one L2.
// A row is P passes of 256 sixteen-channel segments; a register ring of
// R rows (R * P passes) keeps the next rows' loads in flight while one is
// ranked (pass p of a row is refilled with pass p of the row R places on as
// soon as it is unpacked, so every load is issued four passes ahead of its
// use), and a row in the ring is whole, so the token mean and the FP8 scale
// are formed from the registers.  Each 4-block is ranked by the tournament
// and packed by gfx950's packed conversion.
// The 16 channel factors of segment seg (CLACT column norm or weight factor).
__device__ __forceinline__ void seg_factors(const PruneArgs& a, int seg, float (&fv)[16]) {
  const float4* f4 = reinterpret_cast<const float4*>((a.colnorm ? a.colnorm : a.chan_scale) + (size_t)seg * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 q = f4[i];
    fv[4 * i] = q.x; fv[4 * i + 1] = q.y; fv[4 * i + 2] = q.z; fv[4 * i + 3] = q.w;
  }
}

// Ranks the four 4-blocks of one segment of shifted values xh (scores
// |xh| * fv, or |xh|): the 16-bit word of position codes and each block's
// two kept values.
template <bool FAC>
__device__ __forceinline__ uint32_t seg_top2(const float (&xh)[16], const float (&fv)[16], float (&flo)[4],
                                             float (&fhi)[4]) {
  uint32_t meta = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = FAC ? __builtin_fabsf(xh[4 * b + j]) * fv[4 * b + j] : __builtin_fabsf(xh[4 * b + j]);
    meta |= top2of4(sc, xh + 4 * b, flo[b], fhi[b]) << (4 * b);
  }
  return meta;
}

template <int DT, int P, bool FP8, bool FAC>
__global__ void __launch_bounds__(256) k_prune24(PruneArgs a) {
  using T = typename Dt<DT>::T;
  constexpr int R = 4 / P;                   // rows in the ring (four passes)
  constexpr int G = R * P;
  __shared__ double s_red[4];
  __shared__ float s_mx[4];
  const int nseg = a.k / 16;
  const int tid = threadIdx.x;
  const T* x = static_cast<const T*>(a.x);
  auto row_of = [&](int j) -> int {          // the j-th row of this workgroup, or -1
    const long v = (long)j * gridDim.x + blockIdx.x;
    return v < a.t ? xcd_contiguous((int)v, a.t) : -1;
  };
  // a row's buffer descriptor (an absent row reads as zeros)
  auto rsrc_of = [&](int row) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(x) + (size_t)(row < 0 ? 0 : row) * a.k, (short)0,
                                             row < 0 ? 0 : a.k * (int)sizeof(T), kBufferWord3);
  };
  RawSeg<DT, 16> raw[G];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const int row = row_of(rr);
    const auto rs = rsrc_of(row);
#pragma unroll
    for (int p = 0; p < P; ++p) load_raw<DT, 16>(rs, p * 256 + tid, row >= 0 && p * 256 + tid < nseg, raw[rr * P + p]);
  }

  for (int j0 = 0; row_of(j0) >= 0; j0 += R) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int row = row_of(j0 + rr);
      if (row < 0) break;                    // the same for the whole workgroup
      float eta = 0.f;
      if (a.shift_mean) {
        double s = 0.0;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          if (p * 256 + tid < nseg) {
            float v[16];
            unpack_raw<DT, 16>(raw[rr * P + p], a.act, v);
#pragma unroll
            for (int j = 0; j < 16; ++j) s += (double)v[j];
          }
        }
        eta = (float)(block_sum(s, s_red) / (double)a.k);
      } else if (a.eta_given) {
        // a scalar load: kept off the vector-memory counter, whose in-order
        // waits would otherwise hold back on the ring's loads
        eta = ((const __attribute__((address_space(4))) float*)(uintptr_t)a.eta_given)[row];
      }
      if (tid == 0 && a.eta_out) a.eta_out[row] = eta;
      float fp8_inv = 0.f;
      if constexpr (FP8) {
        float mx = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const int seg = p * 256 + tid;
          if (seg < nseg) {
            float v[16], fv[16], flo[4], fhi[4];
            unpack_raw<DT, 16>(raw[rr * P + p], a.act, v);
            if constexpr (FAC) seg_factors(a, seg, fv);
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] -= eta;
            seg_top2<FAC>(v, fv, flo, fhi);
#pragma unroll
            for (int b = 0; b < 4; ++b) mx = fmaxf(mx, fmaxf(__builtin_fabsf(flo[b]), __builtin_fabsf(fhi[b])));
          }
        }
        const float amax = block_max(mx, s_mx);
        float scale;
        fp8_scales(amax, scale, fp8_inv);
        if (tid == 0) a.fp8_scale[row] = scale;
      }
      const int next = row_of(j0 + rr + R);
      const auto rs_next = rsrc_of(next);
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int seg = p * 256 + tid;
        float v[16];
        unpack_raw<DT, 16>(raw[rr * P + p], a.act, v);
        load_raw<DT, 16>(rs_next, seg, next >= 0 && seg < nseg, raw[rr * P + p]);
        if (seg < nseg) {
          float fv[16], flo[4], fhi[4];
          if constexpr (FAC) seg_factors(a, seg, fv);
#pragma unroll
          for (int j = 0; j < 16; ++j) v[j] -= eta;
          const uint32_t meta = seg_top2<FAC>(v, fv, flo, fhi);
          const size_t rowpos = (size_t)(seg / 4) * a.t_pad + row;
          if constexpr (FP8) {
            const uint32_t q01 = fp8_pair(flo[0] * fp8_inv, fhi[0] * fp8_inv) |
                                 (fp8_pair(flo[1] * fp8_inv, fhi[1] * fp8_inv) << 16);
            const uint32_t q23 = fp8_pair(flo[2] * fp8_inv, fhi[2] * fp8_inv) |
                                 (fp8_pair(flo[3] * fp8_inv, fhi[3] * fp8_inv) << 16);
            reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.tiled_vals) + rowpos * 32)[seg % 4] = make_uint2(q01, q23);
          } else {
            reinterpret_cast<uint4*>(static_cast<T*>(a.tiled_vals) + rowpos * 32)[seg % 4] =
                make_uint4(pack2<DT>(flo[0], fhi[0]), pack2<DT>(flo[1], fhi[1]), pack2<DT>(flo[2], fhi[2]),
                           pack2<DT>(flo[3], fhi[3]));
          }
          a.tiled_meta[rowpos * 4 + seg % 4] = (uint16_t)meta;
        }
      }
    }
  }
}

// As many workgroups as the GPU holds at once (CUs x the kernel's
// workgroups per CU, queried once per instantiation), fewer when that leaves
// the rows uneven, and a multiple of the 8 XCDs.
struct Residency {
  hipError_t err;
  int per_gpu;
};
template <int DT, int P, bool FP8, bool FAC>
static hipError_t prune24_launch(const PruneArgs& a, hipStream_t st) {
  static const Residency res = [] {
    int dev = 0, nb = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_prune24<DT, P, FP8, FAC>, 256, 0);
    return Residency{e, (ncu > 0 ? ncu : 1) * (nb > 0 ? nb : 1)};
  }();
  if (res.err != hipSuccess) return res.err;
  const long per = (a.t + (long)res.per_gpu - 1) / res.per_gpu;    // rows per workgroup
  const long grid = ((a.t + per - 1) / per + 7) / 8 * 8;
  hipLaunchKernelGGL((k_prune24<DT, P, FP8, FAC>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int DT, int P>
static hipError_t prune24_p(const PruneArgs& a, hipStream_t st) {
  const bool fac = a.colnorm || a.chan_scale;
  if (a.fp8) return fac ? prune24_launch<DT, P, true, true>(a, st) : prune24_launch<DT, P, true, false>(a, st);
  return fac ? prune24_launch<DT, P, false, true>(a, st) : prune24_launch<DT, P, false, false>(a, st);
}

// The 2:4 operand by blocks of 16 token rows, for calls that form neither a
// token mean nor an FP8 scale in the pass: wave w of a workgroup takes one
// 64-channel step of its 16 rows per pass, lane 4 r + q holding segment q of
// row r, so that the wave's packed values of that step are one contiguous
// 1 KB run of the step-major operand and its position words one whole
// 128-byte line (a workgroup per row writes 64-byte pieces 256 KB apart).
// Workgroup (row block, column group) walks the column group's steps four at
// a time, a four-pass register ring holding the next passes' loads.
template <int DT, bool FAC, int PER>
__global__ void __launch_bounds__(256) k_prune24_rows(PruneArgs a) {
  using T = typename Dt<DT>::T;
  constexpr int G = PER < 4 ? PER : 4;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane >> 2, q = lane & 3;
  const int row = blockIdx.x * 16 + r;
  const bool live = row < a.t;
  const int rowc = live ? row : a.t - 1;                   // rows past t read the last row, store nothing
  const int nsteps = a.k / 64, npass = (nsteps + 3) / 4;
  const int p0 = (int)blockIdx.y * PER, p1 = min(npass, p0 + PER);
  float eta = 0.f;
  if (a.eta_given) eta = a.eta_given[rowc];
  if (blockIdx.y == 0 && wv == 0 && q == 0 && live && a.eta_out) a.eta_out[row] = eta;
  // Descriptors over x and the operand (the host keeps each below 2^31
  // bytes): a load or store at kBufferOutOfRange is dropped, so passes past
  // the column group, steps past k and rows past t need no branch, and the
  // loop's memory counts stay the same on every path.
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.x), (short)0, (int)((size_t)a.t * a.k * sizeof(T)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      a.tiled_vals, (short)0, (int)((size_t)a.t_pad * a.k * sizeof(T) / 2), kBufferWord3);
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      a.tiled_meta, (short)0, (int)((size_t)a.t_pad * (a.k / 16) * 2), kBufferWord3);
  const uint32_t rowoff = (uint32_t)rowc * (uint32_t)a.k * (uint32_t)sizeof(T);
  // pass p's segment of this lane: step 4 p + wv, slot q of its row
  auto load = [&](int p, RawSeg<DT, 16>& raw) {
    const int s = 4 * p + wv;
    const bool ok = p < p1 && s < nsteps;
#pragma unroll
    for (int i = 0; i < RawSeg<DT, 16>::NQ; ++i)
      raw.q[i] = buffer_load16(xrs, ok ? rowoff + (uint32_t)((4 * s + q) * 16 * sizeof(T) + 16 * i) : kBufferOutOfRange);
  };
  // PER passes, unrolled whole: the ring's slots are fixed registers with no
  // loop-carried copies, so each wait counts exactly the loads it needs
  RawSeg<DT, 16> raw[G];
#pragma unroll
  for (int u = 0; u < G; ++u) load(p0 + u, raw[u]);
#pragma unroll
  for (int pb = 0; pb < PER; pb += G) {
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int p = p0 + pb + u;
      float v[16];
      unpack_raw<DT, 16>(raw[u], a.act, v);
      if (pb + u + G < PER) load(p + G, raw[u]);
      const int s = 4 * p + wv;
      const bool ok = live && p < p1 && s < nsteps;
      const int seg = 4 * min(s, nsteps - 1) + q;
      float fv[16], flo[4], fhi[4];
      if constexpr (FAC) seg_factors(a, seg, fv);
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] -= eta;
      const uint32_t meta = seg_top2<FAC>(v, fv, flo, fhi);
      const uint32_t rowpos = (uint32_t)s * (uint32_t)a.t_pad + (uint32_t)row;
      const auto pk = __builtin_bit_cast(
          __attribute__((ext_vector_type(4))) uint32_t,
          make_uint4(pack2<DT>(flo[0], fhi[0]), pack2<DT>(flo[1], fhi[1]), pack2<DT>(flo[2], fhi[2]),
                     pack2<DT>(flo[3], fhi[3])));
      __builtin_amdgcn_raw_buffer_store_b128(pk, vrs, (int)(ok ? rowpos * 64u + 16u * q : kBufferOutOfRange), 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)meta, mrs, (int)(ok ? rowpos * 8u + 2u * q : kBufferOutOfRange), 0, 0);
    }
  }
}

template <int DT, int PER>
static void prune24_rows_per(const PruneArgs& a, dim3 grid, hipStream_t st) {
  if (a.colnorm || a.chan_scale) hipLaunchKernelGGL((k_prune24_rows<DT, true, PER>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_prune24_rows<DT, false, PER>), grid, dim3(256), 0, st, a);
}

template <int DT>
static hipError_t prune24_rows(const PruneArgs& a, hipStream_t st) {
  // about four workgroups per CU: row blocks x column groups of PER passes,
  // PER a power of two up to 16
  const int rbs = (a.t + 15) / 16, npass = (a.k / 64 + 3) / 4;
  const int want = (npass * rbs + 1023) / 1024;            // passes per workgroup for ~1024 workgroups
  int per = 1;
  while (per < want && per < 16) per *= 2;
  const dim3 grid((unsigned)rbs, (unsigned)((npass + per - 1) / per));
  switch (per) {
    case 1: prune24_rows_per<DT, 1>(a, grid, st); break;
    case 2: prune24_rows_per<DT, 2>(a, grid, st); break;
    case 4: prune24_rows_per<DT, 4>(a, grid, st); break;
    case 8: prune24_rows_per<DT, 8>(a, grid, st); break;
    default: prune24_rows_per<DT, 16>(a, grid, st); break;
  }
  return hipGetLastError();
}

// The lean pass applies: 16-bit 2:4 rows of at most 16384 channels, the
// tiled operand the only output.
static bool lean24(int dtype, const PruneArgs& a) {
  return dtype != SPA_F32 && a.m == 4 && a.n == 2 && a.pack == kPackTiled24 && !a.var && !a.nu_out &&
         a.k % 64 == 0 && a.k <= 16384;
}

template <int DT>
static hipError_t prune24_dt(const PruneArgs& a, hipStream_t st) {
  // no token mean or FP8 scale to form from whole rows: blocks of 16 rows
  if (!a.shift_mean && !a.fp8 && (size_t)a.t * a.k * Dt<DT>::bytes < (size_t)kBufferOutOfRange &&
      (size_t)a.t_pad * a.k * Dt<DT>::bytes / 2 < (size_t)kBufferOutOfRange)
    return prune24_rows<DT>(a, st);
  const int passes = (a.k / 16 + 255) / 256;
  return passes <= 1 ? prune24_p<DT, 1>(a, st) : passes <= 2 ? prune24_p<DT, 2>(a, st) : prune24_p<DT, 4>(a, st);
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
  if (lean24(dtype, a)) return dtype == SPA_F16 ? prune24_dt<SPA_F16>(a, st) : prune24_dt<SPA_BF16>(a, st);
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

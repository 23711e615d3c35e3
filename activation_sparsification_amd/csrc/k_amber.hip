// Amber-Pruner channel factor (once per layer, off the timed path).
//
// The activation sparsification guide's weight-aware recipe (s2.2.2): remove
// the weights outside the 0.5th..99.5th percentiles of the whole matrix,
// standardise the rest with their own mean and standard deviation, and take
// channel k's 2-norm over the outputs as its importance:
//   f_k = (sum_{j kept} ((W[j][k] - mean) / std)^2)^(alpha/2).
// The percentiles interpolate linearly, in float64, between the order
// statistics at floor and floor+1 of q/100 * (N - 1); those are found exactly
// by a byte-wise radix select over order-preserving integer keys of the
// weights, one histogram pass per key byte, with the digit choice made on the
// device (no host synchronisation).  Mean, variance and the column sums are
// double-double sums, so the float64 results are the correctly rounded exact
// values in all but pathological cases.
#include "spa_common.h"
#include "spa_launch.h"

namespace spa {

namespace {

constexpr int kRanks = 4;          // order statistics: floor and floor+1 at each percentile
constexpr int kSumBlocks = 1024;   // workgroups of the grid-wide sums

struct AmberState {
  unsigned long long hist[kRanks][256];
  unsigned long long rem[kRanks];   // rank still to skip inside the current prefix
  uint32_t prefix[kRanks];          // key bytes chosen so far
  double g_lo, g_hi;                // interpolation weights
  double lo, hi;                    // the two percentiles
  double mean, var;
  unsigned long long count;
  double part_hi[kSumBlocks], part_lo[kSumBlocks];
  unsigned long long part_n[kSumBlocks];
};

// Order-preserving unsigned key of a stored weight (finite values).
template <int DT>
__device__ __forceinline__ uint32_t weight_key(typename Dt<DT>::T v) {
  if constexpr (DT == SPA_F32) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  } else {
    const uint32_t u = (uint32_t)v;
    return (u & 0x8000u) ? (~u & 0xFFFFu) : (u | 0x8000u);
  }
}
template <int DT>
__device__ __forceinline__ double key_value(uint32_t key) {
  if constexpr (DT == SPA_F32) {
    const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
    return (double)__uint_as_float(u);
  } else {
    const uint32_t u = (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
    return (double)to_f32<DT>((uint16_t)u);
  }
}

__global__ void __launch_bounds__(256) k_amber_init(AmberState* s, unsigned long long r_lo,
                                                    unsigned long long r_hi, unsigned long long n_last, double g_lo,
                                                    double g_hi) {
  for (int i = threadIdx.x; i < kRanks * 256; i += 256) (&s->hist[0][0])[i] = 0ull;
  if (threadIdx.x == 0) {
    const unsigned long long r[kRanks] = {r_lo, r_lo + 1 <= n_last ? r_lo + 1 : n_last, r_hi,
                                          r_hi + 1 <= n_last ? r_hi + 1 : n_last};
    for (int q = 0; q < kRanks; ++q) { s->rem[q] = r[q]; s->prefix[q] = 0u; }
    s->g_lo = g_lo;
    s->g_hi = g_hi;
  }
}

// Histogram of key byte `shift / 8` over the keys whose higher bytes equal
// each rank's prefix.  Per-workgroup counts in LDS, then one global add per bin.
template <int DT>
__global__ void __launch_bounds__(256) k_amber_hist(const typename Dt<DT>::T* __restrict__ w, size_t total,
                                                    AmberState* s, int shift) {
  __shared__ uint32_t h[kRanks][256];
  __shared__ uint32_t pre[kRanks];
  for (int i = threadIdx.x; i < kRanks * 256; i += 256) (&h[0][0])[i] = 0u;
  if (threadIdx.x < kRanks) pre[threadIdx.x] = s->prefix[threadIdx.x];
  __syncthreads();
  const int hs = shift + 8;                                  // bits above the current byte
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const uint32_t key = weight_key<DT>(w[e]);
    const uint32_t d = (key >> shift) & 0xFFu;
    const uint32_t hi = hs >= 32 ? 0u : key >> hs;
#pragma unroll
    for (int q = 0; q < kRanks; ++q)
      if (hi == pre[q]) atomicAdd(&h[q][d], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kRanks * 256; i += 256) {
    const uint32_t c = (&h[0][0])[i];
    if (c) atomicAdd(&(&s->hist[0][0])[i], (unsigned long long)c);
  }
}

// Choose each rank's next key byte from its histogram and clear the histogram
// for the next pass; after the last byte, form the two percentiles.
template <int DT>
__global__ void __launch_bounds__(64) k_amber_select(AmberState* s, int last) {
#pragma clang fp contract(off)
  const int q = threadIdx.x;
  if (q < kRanks) {
    unsigned long long rem = s->rem[q], below = 0ull;
    int d = 255;
    for (int b = 0; b < 256; ++b) {
      const unsigned long long c = s->hist[q][b];
      if (rem < below + c) { d = b; break; }
      below += c;
    }
    s->rem[q] = rem - below;
    s->prefix[q] = (s->prefix[q] << 8) | (uint32_t)d;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kRanks * 256; i += 64) (&s->hist[0][0])[i] = 0ull;
  if (last && threadIdx.x == 0) {
    const double v0 = key_value<DT>(s->prefix[0]), v1 = key_value<DT>(s->prefix[1]);
    const double v2 = key_value<DT>(s->prefix[2]), v3 = key_value<DT>(s->prefix[3]);
    s->lo = v0 + (v1 - v0) * s->g_lo;
    s->hi = v2 + (v3 - v2) * s->g_hi;
  }
}

// Grid-wide double-double sum over the kept weights: of w (pass 0, with the
// count) or of (w - mean)^2 (pass 1); per-workgroup partials, fixed order.
template <int DT>
__global__ void __launch_bounds__(256) k_amber_sum(const typename Dt<DT>::T* __restrict__ w, size_t total,
                                                   AmberState* s, int pass) {
#pragma clang fp contract(off)
  __shared__ double sh[256], sl[256];
  __shared__ unsigned long long sn[256];
  const double lo = s->lo, hi = s->hi, mean = pass ? s->mean : 0.0;
  DD acc{0.0, 0.0};
  unsigned long long n = 0;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const double v = (double)to_f32<DT>(w[e]);
    if (v >= lo && v <= hi) {
      if (pass) {
        const double d = v - mean;
        dd_add(acc, d * d);
      } else {
        dd_add(acc, v);
        ++n;
      }
    }
  }
  sh[threadIdx.x] = acc.hi; sl[threadIdx.x] = acc.lo; sn[threadIdx.x] = n;
  __syncthreads();
  for (int half = 128; half >= 1; half >>= 1) {
    if ((int)threadIdx.x < half) {
      DD a{sh[threadIdx.x], sl[threadIdx.x]};
      dd_merge(a, DD{sh[threadIdx.x + half], sl[threadIdx.x + half]});
      sh[threadIdx.x] = a.hi; sl[threadIdx.x] = a.lo;
      sn[threadIdx.x] += sn[threadIdx.x + half];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    s->part_hi[blockIdx.x] = sh[0];
    s->part_lo[blockIdx.x] = sl[0];
    s->part_n[blockIdx.x] = sn[0];
  }
}

// The workgroup partials combined in a fixed order: four per thread in
// sequence, then a tree over the 256 threads.
__global__ void __launch_bounds__(256) k_amber_reduce(AmberState* s, int nblk, int pass) {
  __shared__ double sh[256], sl[256];
  __shared__ unsigned long long sn[256];
  DD acc{0.0, 0.0};
  unsigned long long n = 0;
  for (int b = threadIdx.x * 4; b < (int)threadIdx.x * 4 + 4 && b < nblk; ++b) {
    dd_merge(acc, DD{s->part_hi[b], s->part_lo[b]});
    n += s->part_n[b];
  }
  sh[threadIdx.x] = acc.hi; sl[threadIdx.x] = acc.lo; sn[threadIdx.x] = n;
  __syncthreads();
  for (int half = 128; half >= 1; half >>= 1) {
    if ((int)threadIdx.x < half) {
      DD a{sh[threadIdx.x], sl[threadIdx.x]};
      dd_merge(a, DD{sh[threadIdx.x + half], sl[threadIdx.x + half]});
      sh[threadIdx.x] = a.hi; sl[threadIdx.x] = a.lo;
      sn[threadIdx.x] += sn[threadIdx.x + half];
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  const double tot = sh[0] + sl[0];
  if (pass == 0) {
    s->count = sn[0];
    s->mean = sn[0] ? tot / (double)sn[0] : 0.0;
  } else {
    s->var = s->count ? tot / (double)s->count : 0.0;
  }
}

// Sum over outputs of each channel's kept (w - mean)^2 (64 channels x 4 row
// groups per workgroup).
template <int DT>
__global__ void __launch_bounds__(256) k_amber_cols(const typename Dt<DT>::T* __restrict__ w, int n_out, int k,
                                                    const AmberState* s, double half_alpha, float* __restrict__ out) {
#pragma clang fp contract(off)
  const double lo = s->lo, hi = s->hi, mean = s->mean, var = s->var;
  bool owner;
  int c;
  const DD acc = column_dd(
      w, n_out, k, [](typename Dt<DT>::T x) { return (double)to_f32<DT>(x); },
      [=](DD& a, double v) {
#pragma clang fp contract(off)
        if (v >= lo && v <= hi) {
          const double d = v - mean;
          dd_add(a, d * d);
        }
      },
      owner, c);
  if (!owner) return;
  const double ss = var > 0.0 ? (acc.hi + acc.lo) / var : 0.0;
  out[c] = (float)pow(ss, half_alpha);
}

template <int DT>
hipError_t amber_impl(const void* wv, int n_out, int k, float alpha, float* out, void* ws, hipStream_t st) {
  using T = typename Dt<DT>::T;
  const T* w = static_cast<const T*>(wv);
  AmberState* s = static_cast<AmberState*>(ws);
  const size_t total = (size_t)n_out * (size_t)k;
  // percentile positions, as q / 100 * (N - 1) in float64
  const double p_lo = 0.5 / 100.0 * (double)(total - 1), p_hi = 99.5 / 100.0 * (double)(total - 1);
  const unsigned long long r_lo = (unsigned long long)p_lo, r_hi = (unsigned long long)p_hi;
  hipLaunchKernelGGL(k_amber_init, dim3(1), dim3(256), 0, st, s, r_lo, r_hi, (unsigned long long)(total - 1),
                     p_lo - (double)r_lo, p_hi - (double)r_hi);
  if (hipError_t e = hipGetLastError()) return e;
  const size_t blocks = (total + 255) / 256;
  const unsigned grid = (unsigned)(blocks < (size_t)kSumBlocks ? blocks : (size_t)kSumBlocks);
  constexpr int kBytes = Dt<DT>::bytes;
  for (int byte = kBytes - 1; byte >= 0; --byte) {
    hipLaunchKernelGGL(k_amber_hist<DT>, dim3(grid), dim3(256), 0, st, w, total, s, 8 * byte);
    hipLaunchKernelGGL(k_amber_select<DT>, dim3(1), dim3(64), 0, st, s, byte == 0 ? 1 : 0);
    if (hipError_t e = hipGetLastError()) return e;
  }
  for (int pass = 0; pass < 2; ++pass) {
    hipLaunchKernelGGL(k_amber_sum<DT>, dim3(grid), dim3(256), 0, st, w, total, s, pass);
    hipLaunchKernelGGL(k_amber_reduce, dim3(1), dim3(256), 0, st, s, (int)grid, pass);
    if (hipError_t e = hipGetLastError()) return e;
  }
  hipLaunchKernelGGL(k_amber_cols<DT>, dim3((k + 63) / 64), dim3(256), 0, st, w, n_out, k, s,
                     0.5 * (double)alpha, out);
  return hipGetLastError();
}

}  // namespace

size_t amber_workspace_bytes() { return (sizeof(AmberState) + 255) & ~size_t(255); }

hipError_t launch_amber(int dtype, const void* w, int n_out, int k, float alpha, float* out, void* ws,
                        hipStream_t st) {
  switch (dtype) {
    case SPA_F32: return amber_impl<SPA_F32>(w, n_out, k, alpha, out, ws, st);
    case SPA_F16: return amber_impl<SPA_F16>(w, n_out, k, alpha, out, ws, st);
    default: return amber_impl<SPA_BF16>(w, n_out, k, alpha, out, ws, st);
  }
}

}  // namespace spa

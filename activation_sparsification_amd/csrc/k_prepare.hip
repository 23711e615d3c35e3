// Weight preparation (once per layer, off the timed path).
//
//   wt[c][j]       = W[j][c]                         channel-major copy
//   chan_scale[c]  = float32((sum_j W[j][c]^2)^(alpha/2))
//   row_sum[j]     = float32(sum_c W[j][c])
//
// The per-channel weight norm is the weight-aware score's factor (WiSparse
// s2.1, eq. (4): it can be formed ahead of time); the row sums carry the
// per-token shift past the pruned product ((x_sparse + eta) W^T =
// x_sparse W^T + eta * W 1, guide s3.1).  Both sums are taken in
// double-double arithmetic so the float64 result is the correctly rounded
// exact sum in all but pathological cases.
#include "spa_common.h"
#include "spa_launch.h"

namespace spa {

template <int DT>
__global__ void __launch_bounds__(256) k_transpose(const typename Dt<DT>::T* __restrict__ w,
                                                   typename Dt<DT>::T* __restrict__ wt, int n_out, int k) {
  using T = typename Dt<DT>::T;
  __shared__ T tile[64][65];
  const int c0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int j = j0 + r, c = c0 + tx;
    if (j < n_out && c < k) tile[r][tx] = w[(size_t)j * k + c];
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int c = c0 + r, j = j0 + tx;
    if (j < n_out && c < k) wt[(size_t)c * n_out + j] = tile[tx][r];
  }
}

// Squares summed down each column (64 columns x 4 row groups per workgroup).
template <int DT>
__global__ void __launch_bounds__(256) k_chan_scale(const typename Dt<DT>::T* __restrict__ w, float* __restrict__ out,
                                                    int n_out, int k, double half_alpha) {
  bool owner;
  int c;
  const DD acc = column_dd(
      w, n_out, k, [](typename Dt<DT>::T x) { return (double)to_f32<DT>(x); },
      [](DD& a, double v) { dd_add(a, v * v); },   // exact: a float32 squared fits in 53 bits
      owner, c);
  if (owner) out[c] = (float)pow(acc.hi + acc.lo, half_alpha);
}

// One workgroup per output row.
template <int DT>
__global__ void __launch_bounds__(256) k_row_sum(const typename Dt<DT>::T* __restrict__ w, float* __restrict__ out,
                                                 int k) {
  __shared__ double s_hi[256], s_lo[256];
  const int j = blockIdx.x;
  DD acc{0.0, 0.0};
  for (int c = threadIdx.x; c < k; c += 256) dd_add(acc, (double)to_f32<DT>(w[(size_t)j * k + c]));
  s_hi[threadIdx.x] = acc.hi;
  s_lo[threadIdx.x] = acc.lo;
  __syncthreads();
  for (int half = 128; half >= 1; half >>= 1) {
    if ((int)threadIdx.x < half) {
      DD a{s_hi[threadIdx.x], s_lo[threadIdx.x]};
      const DD b{s_hi[threadIdx.x + half], s_lo[threadIdx.x + half]};
      dd_merge(a, b);
      s_hi[threadIdx.x] = a.hi;
      s_lo[threadIdx.x] = a.lo;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[j] = (float)(s_hi[0] + s_lo[0]);
}

template <int DT>
static hipError_t prepare_impl(const void* w, int n_out, int k, float alpha, void* wt, float* cs, float* rs,
                               hipStream_t st) {
  using T = typename Dt<DT>::T;
  const T* wp = static_cast<const T*>(w);
  if (wt) {
    dim3 grid((k + 63) / 64, (n_out + 63) / 64);
    hipLaunchKernelGGL(k_transpose<DT>, grid, dim3(256), 0, st, wp, static_cast<T*>(wt), n_out, k);
    if (hipError_t e = hipGetLastError()) return e;
  }
  if (cs) {
    hipLaunchKernelGGL(k_chan_scale<DT>, dim3((k + 63) / 64), dim3(256), 0, st, wp, cs, n_out, k,
                       0.5 * (double)alpha);
    if (hipError_t e = hipGetLastError()) return e;
  }
  if (rs) {
    hipLaunchKernelGGL(k_row_sum<DT>, dim3(n_out), dim3(256), 0, st, wp, rs, k);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

hipError_t launch_prepare(int dtype, const void* w, int n_out, int k, float alpha, void* wt, float* cs, float* rs,
                          hipStream_t st) {
  switch (dtype) {
    case SPA_F32: return prepare_impl<SPA_F32>(w, n_out, k, alpha, wt, cs, rs, st);
    case SPA_F16: return prepare_impl<SPA_F16>(w, n_out, k, alpha, wt, cs, rs, st);
    default: return prepare_impl<SPA_BF16>(w, n_out, k, alpha, wt, cs, rs, st);
  }
}

}  // namespace spa

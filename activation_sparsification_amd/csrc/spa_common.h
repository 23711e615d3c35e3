// Shared device helpers of the N:M activation-pruning library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spa.h"

namespace spa {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Storage dtypes.  16-bit values travel as raw uint16_t bits.
// ---------------------------------------------------------------------------
template <int DT> struct Dt;
template <> struct Dt<SPA_F32> { using T = float; static constexpr int bytes = 4; };
template <> struct Dt<SPA_F16> { using T = uint16_t; static constexpr int bytes = 2; };
template <> struct Dt<SPA_BF16> { using T = uint16_t; static constexpr int bytes = 2; };

__device__ __forceinline__ float bf16_to_f32(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)u);
}
// Round-to-nearest-even float -> bfloat16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Two float32 values as one word of 16-bit values (lo in the low half), each
// rounded to nearest even by gfx950's packed conversion (v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32; the kernels run with float32 denormals preserved, so the
// bf16 result equals f32_to_bf16's for every finite input).
template <int DT> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<SPA_BF16>(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}
template <> __device__ __forceinline__ uint32_t pack2<SPA_F16>(float lo, float hi) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t p = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

template <int DT> __device__ __forceinline__ float to_f32(typename Dt<DT>::T v);
template <> __device__ __forceinline__ float to_f32<SPA_F32>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<SPA_F16>(uint16_t v) { return f16_to_f32(v); }
template <> __device__ __forceinline__ float to_f32<SPA_BF16>(uint16_t v) { return bf16_to_f32(v); }

template <int DT> __device__ __forceinline__ typename Dt<DT>::T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<SPA_F32>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<SPA_F16>(float v) { return (uint16_t)f32_to_f16(v); }
template <> __device__ __forceinline__ uint16_t from_f32<SPA_BF16>(float v) { return (uint16_t)f32_to_bf16(v); }

// Squared ReLU of a stored input value v (already float32): max(v, 0)^2 in
// float32 -- exact for 16-bit v -- rounded back to the storage dtype, so the
// fused path sees what a separate elementwise pass would have stored.
template <int DT>
__device__ __forceinline__ float relu2(float v) {
#pragma clang fp contract(off)
  const float r = v > 0.f ? v : 0.f;
  const float sq = r * r;
  return to_f32<DT>(from_f32<DT>(sq));
}
// The input transform of cfg->act (0: none, 1: squared ReLU); act is
// uniform across the launch.
template <int DT>
__device__ __forceinline__ float apply_act(float v, int act) { return act ? relu2<DT>(v) : v; }

// FP8 (OCP e4m3) codes of two float32 values, rounded to nearest even (the
// gfx950 conversion; values beyond 464 in magnitude are outside the format).
__device__ __forceinline__ uint32_t fp8_pair(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}
// Per-row FP8 scaling: scale = max / 448 and its inverse 448 / max, both
// correctly rounded float32 divisions; a zero row gets 0 for both.
__device__ __forceinline__ void fp8_scales(float amax, float& scale, float& inv) {
  scale = amax > 0.f ? __fdiv_rn(amax, 448.f) : 0.f;
  inv = amax > 0.f ? __fdiv_rn(448.f, amax) : 0.f;
}

// Element e (0..7) of a 16-byte vector of 16-bit values.
template <int DT> __device__ __forceinline__ float elem16(const uint4& v, int e) {
  uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
  return DT == SPA_BF16 ? bf16_to_f32(h) : f16_to_f32(h);
}

// Raw buffer loads (CDNA): a descriptor of base, size in bytes and the gfx9
// format word; a 32-bit byte offset per lane; a load at or past the size
// returns zeros instead of touching memory.
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kBufferOutOfRange = 0x80000000u;   // past every buffer smaller than 2 GiB
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t buffer_load_u16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buffer_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// ---------------------------------------------------------------------------
// Direct global->LDS loads and the waits that order them.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}
// Lane l's 16 (or 4) bytes at sbase + voff land at LDS address lds + 16 l
// (4 l); sbase and lds are wave-uniform.  Issued from asm so that the
// compiler does not add waits of its own before later LDS reads: the kernels
// order these copies with explicit vmcnt waits and the workgroup barrier.
// No register is written, so nothing but LDS bytes is left in flight.  An
// LDS-DMA reading M0 needs one wait state after the M0 write (s_nop 0).
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds)
               : "m0");
}
__device__ __forceinline__ void lds_dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"(sbase), "s"(lds)
               : "m0");
}

// Wait until at most KEEP of this wave's vector-memory operations are
// outstanding (keep != 0), or none (keep == 0).  The gfx9 s_waitcnt field:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at
// their maxima (no wait).
template <int KEEP>
__device__ __forceinline__ void wait_vm(int keep) {
  static_assert(KEEP >= 0 && KEEP < 64, "vmcnt field");
  constexpr int kEnc = 0x0F70 | (KEEP & 15) | ((KEEP >> 4) << 14);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (keep) __builtin_amdgcn_s_waitcnt(kEnc);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Workgroup barrier after this wave's own LDS reads have completed (the stage
// they read is refilled by direct loads right after the barrier).  Vector
// memory is ordered by the explicit wait_vm before it, not here.
__device__ __forceinline__ void bare_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------------------
// The mask arithmetic.  Every helper is a single IEEE operation so that the
// GPU reproduces the reference definition bit for bit.
// ---------------------------------------------------------------------------
// CLACT column energy: one float32 square and one float32 add per token, in
// token order, never fused into an FMA.
__device__ __forceinline__ float clact_accumulate(float acc, float v) {
#pragma clang fp contract(off)
  float sq = v * v;
  return acc + sq;
}
// Correctly rounded float32 square root: the float64 root of a float32 is
// rounded once more without error (53 >= 2*24 + 2).
__device__ __forceinline__ float sqrt_rn(float a) { return (float)__builtin_sqrt((double)a); }


// ---------------------------------------------------------------------------
// The variance factor from a token's dense and masked variances (the guide's
// s3.2): the closed form sqrt(vf / vm) (1 when vm == 0), or, with mode 2, the
// running-average form: r = 0.9 r_in + 0.1 vf, nu = sqrt(r / (vm + 1e-6)),
// the new state written by the one caller that passes `writer`.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float nu_of(double vf, double vm, int mode, const float* r_in, float* r_out, int tok,
                                       bool writer) {
#pragma clang fp contract(off)
  if (mode == 2) {
    const double r = 0.9 * (double)r_in[tok] + 0.1 * vf;
    if (writer) r_out[tok] = (float)r;
    return (float)__builtin_sqrt(r / (vm + 1e-6));
  }
  return vm > 0.0 ? (float)__builtin_sqrt(vf / vm) : 1.f;
}

// ---------------------------------------------------------------------------
// Double-double sums (weight preparation): the float64 result of hi + lo is
// the correctly rounded exact sum in all but pathological cases.
// ---------------------------------------------------------------------------
struct DD { double hi, lo; };
// Error-free transformation: s + e == a + b exactly.
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
#pragma clang fp contract(off)
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}
__device__ __forceinline__ void dd_add(DD& acc, double v) {
#pragma clang fp contract(off)
  double s, e;
  two_sum(acc.hi, v, s, e);
  two_sum(s, acc.lo + e, acc.hi, acc.lo);
}
__device__ __forceinline__ void dd_merge(DD& a, const DD& b) {
#pragma clang fp contract(off)
  double s, e;
  two_sum(a.hi, b.hi, s, e);
  e += a.lo + b.lo;
  two_sum(s, e, a.hi, a.lo);
}

// Column sums of a row-major [n_out][k] matrix: term(v) summed down each
// column in double-double.  Workgroup = 64 columns x 4 row groups (rows
// strided by 4, eight loads in flight per thread); the groups are merged in
// LDS in a fixed order and thread 0..63 receives its column's total.
template <typename T, typename Load, typename Term>
__device__ __forceinline__ DD column_dd(const T* __restrict__ w, int n_out, int k, Load load, Term term,
                                        bool& owner, int& col) {
  __shared__ double s_hi[4][64], s_lo[4][64];
  const int cl = threadIdx.x & 63, rg = threadIdx.x >> 6;
  col = blockIdx.x * 64 + cl;
  DD acc{0.0, 0.0};
  if (col < k) {
    int j = rg;
    for (; j + 28 < n_out; j += 32) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = load(w[(size_t)(j + 4 * u) * k + col]);
#pragma unroll
      for (int u = 0; u < 8; ++u) term(acc, v[u]);
    }
    for (; j < n_out; j += 4) term(acc, load(w[(size_t)j * k + col]));
  }
  s_hi[rg][cl] = acc.hi;
  s_lo[rg][cl] = acc.lo;
  __syncthreads();
  owner = rg == 0 && col < k;
  if (rg == 0) {
    for (int g = 1; g < 4; ++g) dd_merge(acc, DD{s_hi[g][cl], s_lo[g][cl]});
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Wave and workgroup reductions (block_sum: blockDim.x == 256).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// One DPP move of a double (both halves with the same control); lanes outside
// row_mask read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
// Sum over the 64 lanes of a wave in a fixed order, on every lane, with DPP
// moves instead of LDS permutes: pairs and quads (quad_perm), 8 and 16 lanes
// (half-row and row mirrors), then the rows (row_bcast15 into rows 1 and 3,
// row_bcast31 into rows 2 and 3); the total lands in row 3 and lane 63 is
// read back.
__device__ __forceinline__ double wave_sum_dpp(double v) {
  v += dpp_d<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  v += dpp_d<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  v += dpp_d<0x141, 0xF>(v);   // row_half_mirror
  v += dpp_d<0x140, 0xF>(v);   // row_mirror
  v += dpp_d<0x142, 0xA>(v);   // row_bcast15 -> rows 1, 3
  v += dpp_d<0x143, 0xC>(v);   // row_bcast31 -> rows 2, 3
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Maximum of one float per thread (blockDim.x == 256), identical on every thread.
__device__ __forceinline__ float block_max(float v, float* s_tmp /*[4]*/) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) s_tmp[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(s_tmp[0], s_tmp[1]), fmaxf(s_tmp[2], s_tmp[3]));
}

// Sum of one double per thread, identical on every thread.  Fixed order:
// butterfly within each wave, then waves 0..3 in order.
__device__ __forceinline__ double block_sum(double v, double* s_tmp /*[4]*/) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) s_tmp[w] = v;
  __syncthreads();
  return ((s_tmp[0] + s_tmp[1]) + s_tmp[2]) + s_tmp[3];
}

}  // namespace spa

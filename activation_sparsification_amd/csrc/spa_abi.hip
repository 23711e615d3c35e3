// C ABI of the library: argument validation, workspace layout, dispatch.
// Every rejection happens here, before anything is launched.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "spa.h"
#include "spa_check.h"
#include "spa_launch.h"

// Device scratch of sparse_linear_decode_static, one copy per GPU, held until
// the process ends.  The first SPA_STATIC_COUNTER_BYTES hold the split
// counters (zero between calls); the rest is carved like a decode workspace.
// In host code `scratch` names a host-side stand-in: kernels get the device
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[SPA_STATIC_SCRATCH_BYTES];

namespace {

using namespace spa_check;

spa_status hip_status(hipError_t e) { return e == hipSuccess ? SPA_OK : SPA_ERR_HIP; }

// The prefill path; with w8 (FP8 codes of W, one scale per row) the 2:4
// operand is packed as e4m3 codes and the FP8 GEMM runs.
static spa_status prefill_common(const void* x, int32_t t, const spa_weight* w, const spa_prune_cfg* cfg,
                                 const float* eta_in, void* y, uint8_t* idx_out, float* nu_out, void* workspace,
                                 size_t workspace_bytes, void* stream, const uint8_t* w8, const float* w8_scale) {
  if (w->dtype == SPA_F32) return SPA_ERR_UNSUPPORTED;
  // the GEMMs address a 256-row weight tile with 32-bit offsets: 255 * k * 2 B < 4 GiB
  if (w->k > kMaxPrefillK) return SPA_ERR_UNSUPPORTED;
  if (t == 0) return SPA_OK;
  const int k = w->k;
  const PrefillPlan pl = prefill_plan(t, k, w->dtype, cfg);
  if (!workspace || workspace_bytes < pl.bytes || !aligned16(workspace)) return SPA_ERR_INVALID;
  char* base = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool s24 = cfg->n == 2 && cfg->m == 4;
  float* eta_ws = reinterpret_cast<float*>(base + pl.eta);
  float* nu_ptr = nu_out ? nu_out : reinterpret_cast<float*>(base + pl.nu);

  spa::PruneArgs a{};
  a.x = x; a.t = t; a.k = k; a.n = cfg->n; a.m = cfg->m;
  a.var = cfg->var_rescale;
  a.var_in = cfg->var_state;
  a.var_out = cfg->var_state_out;
  a.act = cfg->act;
  a.chan_scale = cfg->score == SPA_SCORE_WEIGHT ? w->chan_scale : nullptr;
  a.eta_given = cfg->shift == SPA_SHIFT_GIVEN ? eta_in : nullptr;
  a.shift_mean = cfg->shift == SPA_SHIFT_TOKEN_MEAN;
  if (cfg->score == SPA_SCORE_CLACT) {
    float* colnorm = reinterpret_cast<float*>(base + pl.colnorm);
    if (cfg->shift == SPA_SHIFT_TOKEN_MEAN) {
      if (hipError_t e = spa::launch_token_mean(w->dtype, x, t, k, cfg->act, eta_ws, st)) return hip_status(e);
      a.eta_given = eta_ws;
      a.shift_mean = 0;
    }
    if (hipError_t e = spa::launch_colnorm(w->dtype, x, cfg->act, a.eta_given, t, k, colnorm, st)) return hip_status(e);
    a.colnorm = colnorm;
  }
  a.eta_out = eta_ws;
  a.nu_out = (cfg->var_rescale || nu_out) ? nu_ptr : nullptr;
  if (s24) {
    a.pack = spa::kPackTiled24 | (idx_out ? spa::kPackVals : 0);
    a.tiled_vals = base + pl.vals;
    a.tiled_meta = reinterpret_cast<uint16_t*>(base + pl.meta);
    a.t_pad = tiled_rows(t);
    a.vals = nullptr;
    a.idx = idx_out;
    if (w8) {
      a.fp8 = 1;
      a.fp8_scale = reinterpret_cast<float*>(base + pl.sx);
    }
  } else {
    a.pack = spa::kPackDense | (idx_out ? spa::kPackVals : 0);
    a.dense = base + pl.vals;
    a.vals = nullptr;
    a.idx = idx_out;
  }
  if (hipError_t e = spa::launch_prune(w->dtype, a, st)) return hip_status(e);

  spa::PrefillArgs g{};
  g.w = w->w;
  g.row_sum = w->row_sum;
  g.a_vals = base + pl.vals;
  g.a_meta = s24 ? reinterpret_cast<const uint16_t*>(base + pl.meta) : nullptr;
  g.t_pad = s24 ? tiled_rows(t) : t;
  g.eta = cfg->shift != SPA_SHIFT_NONE ? eta_ws : nullptr;
  g.nu = cfg->var_rescale ? nu_ptr : nullptr;
  g.y = y;
  g.t = t; g.k = k; g.n_out = w->n_out;
  g.sparse24 = s24 ? 1 : 0;
  if (w8) {
    g.w = w8;
    g.sx = reinterpret_cast<const float*>(base + pl.sx);
    g.sw = w8_scale;
    return hip_status(spa::launch_gemm_fp8(w->dtype, g, st));
  }
  return hip_status(spa::launch_gemm(w->dtype, g, st));
}

}  // namespace

extern "C" {

const char* spa_status_str(spa_status s) {
  switch (s) {
    case SPA_OK: return "ok";
    case SPA_ERR_INVALID: return "invalid argument";
    case SPA_ERR_UNSUPPORTED: return "unsupported combination";
    case SPA_ERR_HIP: return "HIP runtime error";
    case SPA_ERR_SCRATCH: return "needs more device scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

size_t spa_workspace_bytes(int32_t entry, int32_t t, int32_t k, int32_t n_out, int32_t dtype,
                           const spa_prune_cfg* cfg) {
  if (!valid_cfg(cfg) || !valid_dtype(dtype) || !valid_k(k, cfg) || !built_k(k) || t < 0 || t > kMaxDim ||
      n_out < 0 || n_out > kMaxDim)
    return 0;
  switch (entry) {
    case SPA_ENTRY_PRUNE: return prune_ws(t, k, cfg);
    case SPA_ENTRY_DECODE:
      if (t < 1 || t > 32 || n_out < 1) return 0;
      return spa::decode_workspace(t, k, n_out, dtype, cfg->n, cfg->m, cfg->score, cfg->shift, cfg->var_rescale,
                                   nullptr);
    case SPA_ENTRY_PREFILL: return prefill_plan(t, k, dtype, cfg).bytes;
    default: return 0;
  }
}

spa_status spa_prefill_layout(int32_t t, int32_t k, int32_t dtype, const spa_prune_cfg* cfg,
                              spa_operand_layout* out) {
  if (!out || !valid_cfg(cfg) || !valid_dtype(dtype) || !valid_k(k, cfg) || !built_k(k) || t < 0 || t > kMaxDim)
    return SPA_ERR_INVALID;
  const PrefillPlan p = prefill_plan(t, k, dtype, cfg);
  const bool s24 = cfg->n == 2 && cfg->m == 4;
  out->vals = p.vals;
  out->meta = s24 ? p.meta : 0;
  out->eta = p.eta;
  out->scale = s24 ? p.sx : 0;
  out->t_pad = s24 ? tiled_rows(t) : t;
  out->bytes = p.bytes;
  return SPA_OK;
}

spa_status prepare_weight(const void* w, int32_t dtype, int32_t n_out, int32_t k, float alpha, void* wt_out,
                          float* chan_scale_out, float* row_sum_out, void* stream) {
  if (!w || !valid_dtype(dtype) || n_out < 1 || k < 1 || n_out > kMaxDim || k > kMaxDim) return SPA_ERR_INVALID;
  if (!(alpha >= 0.f && alpha <= 16.f)) return SPA_ERR_INVALID;
  return hip_status(spa::launch_prepare(dtype, w, n_out, k, alpha, wt_out, chan_scale_out, row_sum_out,
                                        static_cast<hipStream_t>(stream)));
}

spa_status prune_nm(const void* x, int32_t dtype, int32_t t, int32_t k, const spa_prune_cfg* cfg,
                    const float* chan_scale, const float* eta_in, void* vals_out, uint8_t* idx_out, float* eta_out,
                    float* nu_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_cfg(cfg) || !valid_dtype(dtype) || !valid_k(k, cfg) || t < 0 || t > kMaxDim) return SPA_ERR_INVALID;
  if (t == 0) return SPA_OK;
  if (!x || !vals_out || !aligned16(x) || !aligned16(vals_out)) return SPA_ERR_INVALID;
  if (cfg->score == SPA_SCORE_WEIGHT && !chan_scale) return SPA_ERR_INVALID;
  if (cfg->shift == SPA_SHIFT_GIVEN && !eta_in) return SPA_ERR_INVALID;
  if (!built_k(k)) return SPA_ERR_UNSUPPORTED;
  const size_t need = prune_ws(t, k, cfg);
  if (need && (!workspace || workspace_bytes < need || !aligned16(workspace))) return SPA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);

  spa::PruneArgs a{};
  a.x = x; a.t = t; a.k = k; a.n = cfg->n; a.m = cfg->m;
  a.var = cfg->var_rescale;
  a.var_in = cfg->var_state;
  a.var_out = cfg->var_state_out;
  a.act = cfg->act;
  a.chan_scale = cfg->score == SPA_SCORE_WEIGHT ? chan_scale : nullptr;
  a.eta_given = cfg->shift == SPA_SHIFT_GIVEN ? eta_in : nullptr;
  a.shift_mean = cfg->shift == SPA_SHIFT_TOKEN_MEAN;
  if (cfg->score == SPA_SCORE_CLACT) {
    float* colnorm = reinterpret_cast<float*>(workspace);
    float* eta_ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256((size_t)k * 4));
    const float* eta = a.eta_given;
    if (cfg->shift == SPA_SHIFT_TOKEN_MEAN) {
      if (hipError_t e = spa::launch_token_mean(dtype, x, t, k, cfg->act, eta_ws, st)) return hip_status(e);
      eta = eta_ws;
      a.eta_given = eta_ws;
      a.shift_mean = 0;
    }
    if (hipError_t e = spa::launch_colnorm(dtype, x, cfg->act, eta, t, k, colnorm, st)) return hip_status(e);
    a.colnorm = colnorm;
  }
  a.pack = spa::kPackVals;
  a.vals = vals_out;
  a.idx = idx_out;
  a.eta_out = eta_out;
  a.nu_out = nu_out;
  return hip_status(spa::launch_prune(dtype, a, st));
}

}  // extern "C"

namespace {

// The decode call once its workspace is placed: `base` holds the plan's
// carve-up (a is the plan, offsets relative to base); `counters`, when not
// NULL, replaces the plan's split counters (which must read zero).
spa_status decode_launch(spa::DecodeArgs& a, char* base, unsigned* counters, const void* x, int32_t t,
                         const spa_weight* w, const spa_prune_cfg* cfg, const float* eta_in, void* y,
                         uint8_t* idx_out, float* nu_out, void* stream) {
  auto fix = [&](auto*& ptr) { ptr = reinterpret_cast<std::remove_reference_t<decltype(ptr)>>(base + reinterpret_cast<uintptr_t>(ptr)); };
  fix(a.partial);
  fix(a.stats);
  fix(a.counters);
  fix(a.eta_ws);
  if (spa::decode_on_matrix_cores(t, w->dtype)) fix(a.dense);   // matrix-core path (the dense offset is 0)
  if (counters) a.counters = counters;
  a.x = x;
  a.act = cfg->act;
  a.var_in = cfg->var_state;
  a.var_out = cfg->var_state_out;
  a.wt = w->wt;
  a.w = w->w;
  a.chan_scale = w->chan_scale;
  a.row_sum = w->row_sum;
  a.eta = cfg->shift == SPA_SHIFT_GIVEN ? eta_in : nullptr;
  a.y = y;
  a.idx_out = idx_out;
  a.nu_out = nu_out;
  return hip_status(spa::launch_decode(w->dtype, a, static_cast<hipStream_t>(stream)));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices];

__global__ void __launch_bounds__(256) k_zero_words(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = 0u;
}

// This GPU's scratch: the device address of `scratch` for the current
// device, looked up once per device; its counter region is cleared then, on
// `st`, by a fill kernel (no memset node, so a captured first call is safe).
spa_status scratch_of(hipStream_t st, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SPA_ERR_HIP;
    hipLaunchKernelGGL(k_zero_words, dim3(64), dim3(256), 0, st, static_cast<uint32_t*>(ptr),
                       (uint32_t)(SPA_STATIC_COUNTER_BYTES / 4));
    if (hipGetLastError() != hipSuccess) return SPA_ERR_HIP;
    g_scratch[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch[dev];
  return SPA_OK;
}

}  // namespace

extern "C" {

spa_status sparse_linear_decode(const void* x, int32_t t, const spa_weight* w, const spa_prune_cfg* cfg,
                                const float* eta_in, void* y, uint8_t* idx_out, float* nu_out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (spa_status s = check_linear(x, t, w, cfg, eta_in, y, true)) return s;
  if (w->dtype == SPA_F32 && t > 8) return SPA_ERR_UNSUPPORTED;
  spa::DecodeArgs a{};
  const size_t need = spa::decode_workspace(t, w->k, w->n_out, w->dtype, cfg->n, cfg->m, cfg->score, cfg->shift,
                                            cfg->var_rescale, &a);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SPA_ERR_INVALID;
  return decode_launch(a, static_cast<char*>(workspace), nullptr, x, t, w, cfg, eta_in, y, idx_out, nu_out, stream);
}

spa_status sparse_linear_decode_static(const void* x, int32_t t, const spa_weight* w, const spa_prune_cfg* cfg,
                                       const float* eta_in, void* y, uint8_t* idx_out, float* nu_out, void* stream) {
  if (spa_status s = check_linear(x, t, w, cfg, eta_in, y, true)) return s;
  if (w->dtype == SPA_F32 && t > 8) return SPA_ERR_UNSUPPORTED;
  spa::DecodeArgs a{};
  const size_t need = spa::decode_workspace(t, w->k, w->n_out, w->dtype, cfg->n, cfg->m, cfg->score, cfg->shift,
                                            cfg->var_rescale, &a);
  if (need > SPA_STATIC_SCRATCH_BYTES - SPA_STATIC_COUNTER_BYTES ||
      (size_t)a.tiles * 4 > SPA_STATIC_COUNTER_BYTES)
    return SPA_ERR_SCRATCH;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = nullptr;
  if (spa_status s = scratch_of(st, &base)) return s;
  return decode_launch(a, base + SPA_STATIC_COUNTER_BYTES, reinterpret_cast<unsigned*>(base), x, t, w, cfg, eta_in,
                       y, idx_out, nu_out, stream);
}

spa_status sparse_linear_prefill(const void* x, int32_t t, const spa_weight* w, const spa_prune_cfg* cfg,
                                 const float* eta_in, void* y, uint8_t* idx_out, float* nu_out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (spa_status s = check_linear(x, t, w, cfg, eta_in, y, false)) return s;
  return prefill_common(x, t, w, cfg, eta_in, y, idx_out, nu_out, workspace, workspace_bytes, stream, nullptr,
                        nullptr);
}

spa_status prepare_weight_fp8(const void* w, int32_t dtype, int32_t n_out, int32_t k, uint8_t* codes_out,
                              float* scale_out, void* stream) {
  if (!w || !codes_out || !scale_out || !valid_dtype(dtype)) return SPA_ERR_INVALID;
  if (n_out < 1 || n_out > kMaxDim || k < 1 || k > kMaxDim) return SPA_ERR_INVALID;
  if (!aligned16(w) || !aligned16(codes_out)) return SPA_ERR_INVALID;
  if (dtype == SPA_F32 || k % 8) return SPA_ERR_UNSUPPORTED;      // 16-bit rows in 16-byte pieces
  return hip_status(spa::launch_quant_rows(dtype, w, n_out, k, codes_out, scale_out, static_cast<hipStream_t>(stream)));
}

spa_status sparse_linear_prefill_fp8(const void* x, int32_t t, const spa_weight* w, const uint8_t* w_codes,
                                     const float* w_scale, const spa_prune_cfg* cfg, const float* eta_in, void* y,
                                     uint8_t* idx_out, float* nu_out, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  // check_linear wants the 16-bit weight pointer, which this path does not read
  if (!w || !w_codes || !w_scale || !aligned16(w_codes)) return SPA_ERR_INVALID;
  spa_weight wd = *w;
  wd.w = w_codes;
  if (spa_status s = check_linear(x, t, &wd, cfg, eta_in, y, false)) return s;
  if (cfg->n != 2 || cfg->m != 4) return SPA_ERR_UNSUPPORTED;
  return prefill_common(x, t, &wd, cfg, eta_in, y, idx_out, nu_out, workspace, workspace_bytes, stream, w_codes,
                        w_scale);
}

spa_status spa_eta_calibrate(const void* x, int32_t dtype, int32_t t, int32_t k, const int32_t* token_ids,
                             int32_t vocab, double* sums, uint32_t* counts, void* stream) {
  if (!valid_dtype(dtype) || t < 0 || t > kMaxDim || k < 1 || k > kMaxDim || vocab < 0) return SPA_ERR_INVALID;
  if (t == 0) return SPA_OK;
  if (!x || !aligned16(x) || !token_ids || (vocab > 0 && (!sums || !counts))) return SPA_ERR_INVALID;
  if (k % 16) return SPA_ERR_UNSUPPORTED;                          // rows read in 16-channel pieces
  return hip_status(spa::launch_eta_calibrate(dtype, x, t, k, token_ids, vocab, sums, counts,
                                              static_cast<hipStream_t>(stream)));
}

spa_status spa_eta_table(const double* sums, const uint32_t* counts, int32_t vocab, float* table_out,
                         void* stream) {
  if (vocab < 0) return SPA_ERR_INVALID;
  if (vocab == 0) return SPA_OK;
  if (!sums || !counts || !table_out) return SPA_ERR_INVALID;
  return hip_status(spa::launch_eta_table(sums, counts, vocab, table_out, static_cast<hipStream_t>(stream)));
}

spa_status spa_eta_lookup(const float* table, int32_t vocab, const int32_t* token_ids, int32_t t, float* eta_out,
                          void* stream) {
  if (vocab < 0 || t < 0) return SPA_ERR_INVALID;
  if (t == 0) return SPA_OK;
  if (!token_ids || !eta_out || (vocab > 0 && !table)) return SPA_ERR_INVALID;
  return hip_status(spa::launch_eta_lookup(table, vocab, token_ids, t, eta_out, static_cast<hipStream_t>(stream)));
}

size_t spa_ffn_workspace_bytes(int32_t t, int32_t ffn, int32_t dtype) {
  if (t < 0 || t > kMaxDim || ffn < 64 || ffn > kMaxPrefillK || ffn % 64 || (dtype != SPA_F16 && dtype != SPA_BF16))
    return 0;
  const size_t rows = (size_t)tiled_rows(t);
  return round256(rows * (size_t)(ffn / 2) * 2) + round256(rows * (size_t)(ffn / 16) * 2);
}

spa_status sparse_ffn_relu2_prefill(const void* x, int32_t t, const spa_weight* up, const spa_weight* down,
                                    void* y, uint8_t* idx_out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (!x || !y || !up || !down || t < 0 || t > kMaxDim) return SPA_ERR_INVALID;
  if (up->dtype != down->dtype || !valid_dtype(up->dtype)) return SPA_ERR_INVALID;
  const int hidden = up->k, ffn = up->n_out;
  // ffn holds whole 2:4 blocks; hidden is any positive width
  if (hidden < 1 || hidden > kMaxDim || ffn < 4 || ffn > kMaxDim || ffn % 4 || down->k != ffn)
    return SPA_ERR_INVALID;
  if (down->n_out < 1 || down->n_out > kMaxDim) return SPA_ERR_INVALID;
  if (!up->w || !down->w || !aligned16(up->w) || !aligned16(down->w) || !aligned16(x) || !aligned16(y))
    return SPA_ERR_INVALID;
  if (idx_out && !aligned16(idx_out)) return SPA_ERR_INVALID;
  // built for whole 64-channel GEMM steps and 32-bit tile offsets
  if (up->dtype == SPA_F32 || hidden % 64 || ffn % 64 || hidden > kMaxPrefillK || ffn > kMaxPrefillK)
    return SPA_ERR_UNSUPPORTED;
  if (t == 0) return SPA_OK;
  const size_t need = spa_ffn_workspace_bytes(t, ffn, up->dtype);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SPA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int t_pad = tiled_rows(t);
  char* base = static_cast<char*>(workspace);
  void* vals = base;
  uint16_t* meta = reinterpret_cast<uint16_t*>(base + round256((size_t)t_pad * (size_t)(ffn / 2) * 2));

  spa::PrefillArgs u{};
  u.w = up->w;
  u.a_vals = x;
  u.t = t; u.k = hidden; u.n_out = ffn;
  u.sparse24 = 0;
  u.out_vals = vals;
  u.out_meta = meta;
  u.out_t_pad = t_pad;
  u.out_idx = idx_out;
  if (hipError_t e = spa::launch_ffn_up(up->dtype, u, st)) return hip_status(e);

  spa::PrefillArgs g{};
  g.w = down->w;
  g.a_vals = vals;
  g.a_meta = meta;
  g.t_pad = t_pad;
  g.y = y;
  g.t = t; g.k = ffn; g.n_out = down->n_out;
  g.sparse24 = 1;
  return hip_status(spa::launch_gemm(down->dtype, g, st));
}

size_t spa_amber_workspace_bytes(void) { return spa::amber_workspace_bytes(); }

spa_status prepare_amber(const void* w, int32_t dtype, int32_t n_out, int32_t k, float alpha, float* chan_scale_out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!w || !chan_scale_out || !valid_dtype(dtype)) return SPA_ERR_INVALID;
  if (n_out < 1 || k < 1 || n_out > kMaxDim || k > kMaxDim) return SPA_ERR_INVALID;
  if (!(alpha >= 0.f && alpha <= 16.f)) return SPA_ERR_INVALID;
  if (!aligned16(w) || !workspace || !aligned16(workspace) || workspace_bytes < spa::amber_workspace_bytes())
    return SPA_ERR_INVALID;
  return hip_status(spa::launch_amber(dtype, w, n_out, k, alpha, chan_scale_out, workspace,
                                      static_cast<hipStream_t>(stream)));
}

size_t spa_meta_row_bytes(int32_t k, int32_t n, int32_t m, int32_t format) {
  if (!valid_meta(k, n, m, format)) return 0;
  return (size_t)4 * (((int64_t)(k / m) * spa::meta_width(n, m, format) + 31) / 32);
}

spa_status spa_encode_meta(const uint8_t* idx, int32_t t, int32_t k, int32_t n, int32_t m, int32_t format,
                           void* codes, void* stream) {
  if (!valid_meta(k, n, m, format) || t < 0 || t > kMaxDim) return SPA_ERR_INVALID;
  if (t == 0 || spa_meta_row_bytes(k, n, m, format) == 0) return SPA_OK;
  if (!idx || !codes || !aligned16(idx) || !aligned16(codes)) return SPA_ERR_INVALID;
  return hip_status(spa::launch_meta(true, idx, nullptr, static_cast<uint32_t*>(codes), t, k, n, m, format,
                                     static_cast<hipStream_t>(stream)));
}

spa_status spa_decode_meta(const void* codes, int32_t t, int32_t k, int32_t n, int32_t m, int32_t format,
                           uint8_t* idx_out, void* stream) {
  if (!valid_meta(k, n, m, format) || t < 0 || t > kMaxDim) return SPA_ERR_INVALID;
  if (t == 0) return SPA_OK;
  const bool has_codes = spa_meta_row_bytes(k, n, m, format) > 0;
  if (!idx_out || !aligned16(idx_out) || (has_codes && (!codes || !aligned16(codes)))) return SPA_ERR_INVALID;
  return hip_status(spa::launch_meta(false, nullptr, idx_out,
                                     const_cast<uint32_t*>(static_cast<const uint32_t*>(codes)), t, k, n, m,
                                     format, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

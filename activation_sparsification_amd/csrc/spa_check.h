// The C ABI's common argument checks and prefill workspace layout, in plain
// C++ (no HIP types), so that the library and a host-only sanitizer build run
// the same code.  The entry points call these before anything is launched.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "spa.h"
#include "spa_plan.h"

namespace spa_check {

constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr int64_t kMaxPrefillK = int64_t(1) << 23;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int dtype_bytes(int dt) { return dt == SPA_F32 ? 4 : 2; }
inline bool valid_dtype(int dt) { return dt == SPA_F32 || dt == SPA_F16 || dt == SPA_BF16; }

inline bool valid_cfg(const spa_prune_cfg* c) {
  if (!c) return false;
  if (c->m != 4 && c->m != 8 && c->m != 16 && c->m != 32) return false;
  if (c->n < 1 || c->n > c->m) return false;
  if (c->score < SPA_SCORE_MAGNITUDE || c->score > SPA_SCORE_CLACT) return false;
  if (c->shift < SPA_SHIFT_NONE || c->shift > SPA_SHIFT_GIVEN) return false;
  if (c->var_rescale < 0 || c->var_rescale > 2) return false;
  if (c->var_rescale == 2 && (!c->var_state || !c->var_state_out || c->var_state == c->var_state_out)) return false;
  if (c->act != SPA_ACT_NONE && c->act != SPA_ACT_RELU2) return false;
  return true;
}

// k must hold whole m-blocks (anything else is an invalid argument) ...
inline bool valid_k(int64_t k, const spa_prune_cfg* c) { return k >= c->m && k <= kMaxDim && k % c->m == 0; }
// ... and, to be built, whole 16-channel segments of the pruning pass (a valid
// k that is not is an unbuilt combination: 2:4 or 4:8 with k = 36, say).
inline bool built_k(int64_t k) { return k % 16 == 0; }


inline size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

// ---- prune workspace: [colnorm k f32][eta t f32] (CLACT only) ----
inline size_t prune_ws(int t, int k, const spa_prune_cfg* c) {
  if (c->score != SPA_SCORE_CLACT) return 0;
  return round256((size_t)k * 4) + round256((size_t)t * 4);
}

// ---- prefill workspace ----
struct PrefillPlan {
  size_t vals, meta, eta, nu, colnorm, sx, bytes;
};
// Rows of the 2:4 tiled operand are padded to the GEMM's 256-token tile.
inline int tiled_rows(int t) { return (t + 255) / 256 * 256; }

inline PrefillPlan prefill_plan(int t, int k, int dtype, const spa_prune_cfg* c) {
  PrefillPlan p{};
  const bool s24 = c->n == 2 && c->m == 4;
  const size_t rows = s24 ? (size_t)tiled_rows(t) : (size_t)t;
  size_t off = 0;
  p.vals = off; off += round256(rows * (s24 ? k / 2 : k) * dtype_bytes(dtype));
  p.meta = off; off += s24 ? round256(rows * (k / 16) * 2) : 0;
  p.eta = off; off += round256((size_t)t * 4);
  p.nu = off; off += round256((size_t)t * 4);
  p.colnorm = off; off += c->score == SPA_SCORE_CLACT ? round256((size_t)k * 4) : 0;
  p.sx = off; off += s24 ? round256((size_t)t * 4) : 0;    // FP8 path: per-token scales
  p.bytes = off;
  return p;
}

inline spa_status check_linear(const void* x, int32_t t, const spa_weight* w, const spa_prune_cfg* cfg,
                               const float* eta_in, const void* y, bool decode) {
  if (!x || !y || !w || !valid_cfg(cfg)) return SPA_ERR_INVALID;
  if (!valid_dtype(w->dtype)) return SPA_ERR_INVALID;
  if (decode ? (t < 1 || t > 32) : (t < 0 || t > kMaxDim)) return SPA_ERR_INVALID;
  if (w->n_out < 1 || w->n_out > kMaxDim || !valid_k(w->k, cfg)) return SPA_ERR_INVALID;
  if (!aligned16(x) || !aligned16(y)) return SPA_ERR_INVALID;
  if (cfg->score == SPA_SCORE_WEIGHT && !w->chan_scale) return SPA_ERR_INVALID;
  if (cfg->shift == SPA_SHIFT_GIVEN && !eta_in) return SPA_ERR_INVALID;
  if (cfg->shift != SPA_SHIFT_NONE && !w->row_sum) return SPA_ERR_INVALID;
  // the matrix-core decode reads the row-major weight, every other decode
  // the channel-major copy
  const bool reads_wt = decode && !spa::decode_on_matrix_cores(t, w->dtype);
  const void* need = reads_wt ? w->wt : w->w;
  if (!need || !aligned16(need)) return SPA_ERR_INVALID;
  // valid, but outside what the kernels are built for
  if (!built_k(w->k)) return SPA_ERR_UNSUPPORTED;
  if (reads_wt && w->n_out % (16 / dtype_bytes(w->dtype))) return SPA_ERR_UNSUPPORTED;   // 16-byte weight rows
  if (!decode && w->k % 64) return SPA_ERR_UNSUPPORTED;                                   // whole GEMM k steps
  return SPA_OK;
}

inline bool valid_meta(int64_t k, int32_t n, int32_t m, int32_t format) {
  if (m != 4 && m != 8 && m != 16 && m != 32) return false;
  if (n < 1 || n > m) return false;
  if (k < m || k > kMaxDim || k % m) return false;
  return format == SPA_META_BITMAP || format == SPA_META_COMB;
}

}  // namespace spa_check

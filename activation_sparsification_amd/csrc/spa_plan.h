// Decode work split and workspace carve-up (host), and the row-list slot rule
// the fused decode kernel uses (host and device).
//
// Plain C++ with no HIP types, so the same code runs in the library and in a
// host-only check that replays every workgroup's list against its LDS bounds.
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define SPA_PLAN_HD __host__ __device__ __forceinline__
#else
#define SPA_PLAN_HD inline
#endif

namespace spa {

// dtype codes, as in spa.h
constexpr int kPlanF32 = 0;

// Buffer descriptors address at most this many bytes (offsets are 32-bit and
// this value itself reads as out of range).
constexpr uint32_t kPlanBufferLimit = 0x80000000u;

// One-token kernel: 512-column tiles, 8 waves, a channel split covers at most
// 2048 channels.
constexpr int kT1Waves = 8, kT1Threads = kT1Waves * 64, kT1Cols = 512, kT1MaxChan = 2048, kT1MaxSplits = 16;
// Matrix-core path: channels per workgroup of its pruning pass, 64-channel
// steps per ring stage.
constexpr int kPruneChan = 256, kMmSteps = 4;
// Fused kernel: LDS bytes for its row list (row index + one float32
// coefficient per token per entry).
constexpr int kFusedListBytes = 55296;

// The one-token kernel: 16-bit weights small enough for 32-bit buffer
// offsets and at least eight 512-column tiles.
SPA_PLAN_HD bool t1_kernel(int t, int dtype, int k, int n_out) {
  return t == 1 && dtype != kPlanF32 && n_out >= 8 * kT1Cols &&
         (uint64_t)k * (uint64_t)n_out * 2u < (uint64_t)kPlanBufferLimit;
}

// The decode path for t tokens of a dtype: two or more tokens of a 16-bit
// type run on the matrix cores over the row-major weight; one token, and
// float32, stream the channel-major copy.  With two tokens the union of kept
// rows is already about 1 - (1 - n/m)^2 of the weight (three quarters at
// 8:16), so reading all of W at the matrix cores' rate beats gathering the
// union rows: 2 and 4 tokens at the 14336 x 4096 layer took 30.4 us against
// 38.1 and 50.9 us streamed, 2 and 4 tokens of the 4096 x 14336 CLACT layer
// 27.7 us against 43.0 and 119 us.  The planner, the argument check and the
// launcher all decide by this one function, so the workspace carve-up, the
// weight that must be present and the kernels launched cannot disagree.
SPA_PLAN_HD constexpr bool decode_on_matrix_cores(int t, int dtype) { return t > 1 && dtype != kPlanF32; }

// Waves per workgroup of the fused kernel: 8 for the light cases, 4 (so each
// wave may hold up to 512 registers) when several tokens or 32-wide blocks
// are ranked per lane.
SPA_PLAN_HD constexpr int fused_waves_of(int m, int tok) { return (tok >= 2 || m >= 32) ? 4 : 8; }

// Token count the fused kernel is instantiated for.
SPA_PLAN_HD constexpr int fused_tok_of(int t) { return t <= 1 ? 1 : t <= 2 ? 2 : t <= 4 ? 4 : 8; }

// Fused kernel, one token: thread `tid` of pass `base`'s workgroup-wide list
// writes its block's n kept rows at slots [slot, slot + n).  `base` is the
// number of entries the earlier passes listed (every block lists exactly n
// rows with one token), so the slots of a pass follow those of the last.
SPA_PLAN_HD int one_token_list_slot(int base, int tid, int n) { return base + tid * n; }

struct DecodePlan {
  int tiles = 0, splits = 0, k_len = 0, col_tile = 0;
  int chunks = 0;        // matrix-core path: channel chunks of the pruning pass
  int list_cap = 0;      // fused path: LDS list entries per workgroup
  int chunk_blocks = 0;  // fused path: m-blocks per workgroup
  // workspace offsets (bytes); unused ones stay 0
  size_t partial = 0, stats = 0, counters = 0, eta = 0, dense = 0;
  size_t bytes = 0;
};

inline DecodePlan plan_decode(int t, int k, int n_out, int dtype, int n, int m, int var) {
  DecodePlan p;
  const bool fused = !decode_on_matrix_cores(t, dtype);
  size_t bytes = 0;
  auto carve = [&](size_t nbytes) { size_t off = bytes; bytes += (nbytes + 255) & ~(size_t)255; return off; };
  if (t1_kernel(t, dtype, k, n_out)) {
    // 512-column tiles (1 KB of each kept row per load instruction); channel
    // splits until about 224 workgroups run, but at most kT1MaxSplits, so the
    // last arrival reads every split's partial in one batch of loads (28
    // splits took two round trips: 21.0 against 19.3 us for a 4096-column
    // output); each split at most kT1MaxChan channels, the partial traffic
    // near 5 % of the weight bytes
    p.col_tile = kT1Cols;
    p.tiles = (n_out + p.col_tile - 1) / p.col_tile;
    const int blocks = k / m;
    int sp = 224 / p.tiles > 1 ? 224 / p.tiles : 1;
    if (sp > kT1MaxSplits) sp = kT1MaxSplits;
    const double wbytes = (double)k * n / m * n_out * 2.0;
    const int max_by_traffic = (int)(0.05 * wbytes / (8.0 * n_out));
    if (sp > max_by_traffic) sp = max_by_traffic > 1 ? max_by_traffic : 1;
    if (sp > blocks) sp = blocks;
    int bl = (blocks + sp - 1) / sp;
    if (bl * m > kT1MaxChan) bl = kT1MaxChan / m;
    p.k_len = bl * m;
    p.splits = (blocks + bl - 1) / bl;
    p.partial = carve((size_t)p.splits * n_out * 4);
    p.stats = carve(var ? (size_t)p.tiles * p.splits * 4 * 8 : 0);
    p.counters = carve((size_t)p.tiles * 4);
    p.eta = carve(4);
  } else if (fused) {
    // 8 lanes x one 16-byte load = one 128-byte cache line of every listed row
    const int cpl = dtype == kPlanF32 ? 4 : 8;
    p.col_tile = 8 * cpl;
    p.tiles = (n_out + p.col_tile - 1) / p.col_tile;
    // split the channels only when the column tiles alone cannot fill the 256
    // CUs; each wave keeps at least one block, and the partial traffic stays
    // near 5 % of the weight bytes
    const int blocks = k / m;
    int sp = p.tiles >= 192 ? 1 : (256 + p.tiles - 1) / p.tiles;
    const int max_by_waves = blocks / 8 > 1 ? blocks / 8 : 1;
    const double wbytes = (double)k * n / m * n_out * 2.0;
    const int max_by_traffic = (int)(0.05 * wbytes / (8.0 * t * n_out));
    if (sp > max_by_waves) sp = max_by_waves;
    if (sp > max_by_traffic) sp = max_by_traffic > 1 ? max_by_traffic : 1;
    // the workgroup's row list lives in LDS
    const int tok = fused_tok_of(t);
    const int per_block = m < n * t ? m : n * t;          // union rows one block can contribute
    const int max_entries = kFusedListBytes / (4 * (1 + tok));
    const int max_blocks = max_entries / per_block > 1 ? max_entries / per_block : 1;
    int bl = (blocks + sp - 1) / sp;
    if (bl > max_blocks) bl = max_blocks;
    p.k_len = bl * m;
    p.splits = (k + p.k_len - 1) / p.k_len;
    p.list_cap = bl * per_block;
    p.chunk_blocks = bl;
    p.partial = carve((size_t)p.splits * t * n_out * 4);
    p.stats = carve(var ? (size_t)p.tiles * p.splits * t * 4 * 8 : 0);
    p.counters = carve((size_t)p.tiles * 4);
    p.eta = carve((size_t)t * 4);
  } else {
    // matrix-core path: prune once into masked rows (channel chunks of
    // kPruneChan), then one pass over w by 64-row tiles, split over k until
    // about 256 workgroups run; from 192 tiles on, no split (one round of
    // workgroups and no hand-off: 224 tiles x 2 splits, 1.75 rounds on 256
    // CUs, took 29.4-29.9 us at 2 and 4 tokens of the 14336 x 4096 layer,
    // 224 unsplit tiles 26.0-26.1 us)
    p.tiles = (n_out + 63) / 64;
    const int nsteps = (k + 63) / 64;
    int sp = p.tiles >= 192 ? 1 : (256 + p.tiles - 1) / p.tiles;
    if (sp > nsteps) sp = nsteps;
    const int sps = (nsteps + sp - 1) / sp;
    p.k_len = sps * 64;
    p.splits = (nsteps + sps - 1) / sps;
    p.chunks = (k + kPruneChan - 1) / kPruneChan;
    // fragment order; at least kMmSteps steps, since the matrix-core pass
    // reads them kMmSteps at a time
    p.dense = carve((size_t)(nsteps > kMmSteps ? nsteps : kMmSteps) * ((t + 15) / 16) * 2048);
    p.stats = carve(var ? (size_t)p.chunks * t * 4 * 8 : 0);
    p.eta = carve((size_t)t * 4);
    p.partial = carve(p.splits > 1 ? (size_t)p.splits * t * n_out * 4 : 0);
    p.counters = carve((size_t)p.tiles * 4);
  }
  p.bytes = bytes;
  return p;
}

}  // namespace spa

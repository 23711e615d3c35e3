// Host-side launchers of the kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spa {

hipError_t launch_prepare(int dtype, const void* w, int n_out, int k, float alpha, void* wt, float* cs, float* rs,
                          hipStream_t st);

// ---- pruning pass (one workgroup per token row) ----
enum PackFormat : int {
  kPackVals = 1,    // vals[t][k*n/m] (dtype) + optional idx[t][k*n/m] (uint8)
  kPackTiled24 = 2, // 2:4 only, the prefill GEMM's layout: per 64-channel step kt, rows padded to
                    // t_pad: vals[kt][t_pad][32] (dtype) and meta[kt][t_pad][4] (uint16, one
                    // nibble lo | hi << 2 per block, four blocks per word)
  kPackDense = 4,   // masked dense rows xm[t][k] (dtype), zeros at pruned channels
};

struct PruneArgs {
  const void* x;
  const float* chan_scale;   // weight score factor, or NULL
  const float* colnorm;      // CLACT factor (from launch_colnorm), or NULL
  const float* eta_given;    // precomputed / caller shift, or NULL
  int t, k, n, m;
  int shift_mean;            // compute the token mean in-kernel
  int act;                   // input transform (SPA_ACT_*)
  int var;                   // 0, 1 (closed form) or 2 (running average)
  const float* var_in;       // var == 2: state [t]
  float* var_out;            // var == 2: new state [t]
  int pack;                  // PackFormat bits
  void* vals;                // kPackVals
  uint8_t* idx;              // kPackVals, may be NULL
  void* tiled_vals;          // kPackTiled24
  uint16_t* tiled_meta;      // kPackTiled24
  int t_pad;                 // kPackTiled24: rows per step (t rounded up to the GEMM tile)
  int fp8;                   // kPackTiled24: kept values as e4m3 codes (32 bytes per row and step)
  float* fp8_scale;          // fp8: per-token scale max|x_hat| / 448, [t]
  void* dense;               // kPackDense
  float* eta_out;            // may be NULL
  float* nu_out;             // may be NULL
};
hipError_t launch_prune(int dtype, const PruneArgs& a, hipStream_t st);
hipError_t launch_token_mean(int dtype, const void* x, int t, int k, int act, float* eta, hipStream_t st);
hipError_t launch_colnorm(int dtype, const void* x, int act, const float* eta, int t, int k, float* c,
                          hipStream_t st);

// ---- decode ----
struct DecodeArgs {
  const void* x;
  const void* wt;            // [k][n_out] channel-major (one token, and float32)
  const void* w;             // [n_out][k] row-major (16-bit, t >= 2)
  const float* chan_scale;
  const float* row_sum;
  const float* eta;          // precomputed or caller-given shift, or NULL
  void* y;
  uint8_t* idx_out;
  float* nu_out;
  int t, k, n_out, n, m;
  int score;                 // SPA_SCORE_*
  int shift;                 // SPA_SHIFT_*
  int var;                   // 0, 1 (closed form) or 2 (running average)
  const float* var_in;       // var == 2: state [t]
  float* var_out;            // var == 2: new state [t]
  int act;                   // input transform (SPA_ACT_*)
  // workspace carve-up
  float* partial;            // fused: [splits][t][n_out]
  double* stats;             // fused: [tiles][splits][t][4]; matrix-core: [t][4][chunks]
  unsigned* counters;        // fused: [tiles]
  void* dense;               // matrix-core path: masked rows [t][k] (dtype)
  float* eta_ws;             // [t]
  int tiles, splits, k_len, col_tile;
  int chunks;                // matrix-core path: channel chunks of the pruning pass
  int list_cap;              // fused path: LDS list entries per wave
  int chunk_blocks;          // fused path: m-blocks a wave selects and streams at a time
};
size_t decode_workspace(int t, int k, int n_out, int dtype, int n, int m, int score, int shift, int var,
                        DecodeArgs* plan);
hipError_t launch_decode(int dtype, DecodeArgs& a, hipStream_t st);

// ---- static shift table ----
hipError_t launch_eta_calibrate(int dtype, const void* x, int t, int k, const int32_t* ids, int vocab, double* sums,
                                uint32_t* counts, hipStream_t st);
hipError_t launch_eta_table(const double* sums, const uint32_t* counts, int vocab, float* table, hipStream_t st);
hipError_t launch_eta_lookup(const float* table, int vocab, const int32_t* ids, int t, float* eta, hipStream_t st);

// ---- Amber-Pruner channel factor ----
size_t amber_workspace_bytes();
hipError_t launch_amber(int dtype, const void* w, int n_out, int k, float alpha, float* out, void* ws,
                        hipStream_t st);

// ---- compact block metadata ----
int meta_width(int n, int m, int format);
hipError_t launch_meta(bool encode, const uint8_t* idx, uint8_t* idx_out, uint32_t* codes, int t, int k, int n,
                       int m, int format, hipStream_t st);

// ---- prefill ----
struct PrefillArgs {
  const void* w;             // [n_out][k]
  const float* row_sum;
  const void* a_vals;        // 2:4: tiled packed values (kPackTiled24); other n:m: masked dense [t][k]
  const uint16_t* a_meta;    // 2:4 only: tiled position words
  int t_pad;                 // 2:4 only: rows per step of the tiled layout
  const float* eta;          // [t] or NULL
  const float* nu;           // [t] or NULL
  void* y;
  int t, k, n_out;
  int sparse24;
  // dense GEMM with the squared-ReLU epilogue (launch_ffn_up): the output is
  // not stored; max(u, 0)^2 is pruned 2:4 and packed in the tiled layout
  void* out_vals;            // [n_out/64][out_t_pad][32] dtype
  uint16_t* out_meta;        // [n_out/64][out_t_pad][4]
  int out_t_pad;
  uint8_t* out_idx;          // [t][n_out/2] in-block positions, or NULL
  // FP8 2:4 GEMM (launch_gemm_fp8): a_vals holds e4m3 codes, w is [n_out][k]
  // e4m3 codes; y = sx[i] * sw[j] * acc (* nu) + eta * row_sum
  const float* sx;           // [t]
  const float* sw;           // [n_out]
  // 2:4 GEMM: the output columns [col0, col1) this launch covers (launch_gemm sets them)
  int col0, col1;
};
hipError_t launch_gemm(int dtype, const PrefillArgs& a, hipStream_t st);
hipError_t launch_ffn_up(int dtype, const PrefillArgs& a, hipStream_t st);
hipError_t launch_gemm_fp8(int dtype, const PrefillArgs& a, hipStream_t st);
hipError_t launch_quant_rows(int dtype, const void* w, int n_out, int k, uint8_t* codes, float* scale,
                             hipStream_t st);

}  // namespace spa

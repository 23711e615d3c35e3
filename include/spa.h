/*
 * spa.h -- C ABI of the MI355X (gfx950) library for input-adaptive N:M
 * activation pruning fused with the linear layer that consumes it.
 *
 * For each token x (a row of X[t][k]) and a linear layer y = x W^T with
 * W[n_out][k]:
 *
 *   x        the layer input, or, with cfg->act == SPA_ACT_RELU2, the
 *            squared ReLU of the given pre-activation u: x_k = max(u_k, 0)^2
 *            in float32 (exact for 16-bit u) rounded to dtype to nearest
 *            even -- the value a separate elementwise pass would store
 *            ("Accelerating Transformer training and inference with 2:4
 *            sparsity and Squared-ReLU" s2.2 defines the activation, s3.1
 *            fuses it into the kernel that prunes and packs);
 *   eta      per-token shift: 0, the token mean (dynamic per-token shift,
 *            "Activation sparsification: a dynamic pruning method for
 *            efficient LLM inference" s3.1), or a caller-given value (the
 *            static variant of the same section);
 *   x_hat    = x - eta, one float32 subtraction;
 *   score_k  = |x_hat_k| * f_k with f_k = 1 (magnitude, same guide s2.2.1),
 *            f_k = ||W[:,k]||_2^alpha (weight-aware, "LLM inference
 *            optimisation: WiSparse activation sparsification explained"
 *            s2.1 eq. (4)), or f_k = sqrt(sum over the call's tokens of
 *            x_hat_pk^2) (cosine-loss CLACT score, guide s2.2.3; the per-row
 *            factor of that score cannot change an in-block ranking);
 *   mask     keep the n largest scores of every m consecutive channels
 *            (guide s2.1); equal scores go to the lower channel index, so
 *            exactly n are kept per block;
 *   nu       optional variance rescale per token (guide s3.2): the closed
 *            form sqrt(Var[x_hat] / Var[x_hat * mask]) (1 when the
 *            denominator is 0), or its running-average form: a caller-held
 *            state r per token, r' = 0.9 r + 0.1 Var[x_hat] (written to
 *            var_state_out), nu = sqrt(r' / (Var[x_hat * mask] + 1e-6));
 *   y        = nu * (x_hat * mask) W^T + eta * (W 1), which equals the
 *            guide's (x_sparse + eta) W^T without reading pruned rows of W.
 *
 * Numerics of the mask: eta is the float64 sum rounded to float64, divided
 * by k in float64, rounded to float32; scores are single float32 products;
 * CLACT sums squares in float32 over tokens in ascending order (no fused
 * multiply-add) and takes a correctly rounded square root.  Masks, packed
 * values and indices are therefore reproducible bit for bit.
 *
 * Conventions for every entry point:
 *  - Pointers marked [device] are device memory owned by the caller; the
 *    library never allocates, frees or keeps them.  Host pointers (the
 *    config and weight descriptors) are read during the call only.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream) and performs no host synchronisation.
 *  - Return codes only: SPA_ERR_INVALID is returned before anything is
 *    launched when an argument is rejected; SPA_ERR_HIP when a launch fails.
 *  - Device buffers must be 16-byte aligned; rows are dense (no padding).
 *  - dtype is one of SPA_F32, SPA_F16, SPA_BF16 and applies to x, w, wt,
 *    vals and y alike.  Accumulation is float32.
 *  - Inputs must be finite.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef SPA_H_
#define SPA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spa_status {
  SPA_OK = 0,
  SPA_ERR_INVALID = 1,      /* rejected argument; nothing launched */
  SPA_ERR_UNSUPPORTED = 2,  /* valid combination the library does not implement */
  SPA_ERR_HIP = 3,          /* a HIP launch or runtime call failed */
  SPA_ERR_SCRATCH = 4       /* sparse_linear_decode_static: the call needs more
                               than the static scratch buffer holds */
} spa_status;

/* Size of the per-GPU device scratch of sparse_linear_decode_static (held
 * from its first call on a GPU until the process ends), and of its leading
 * split-counter region. */
#define SPA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
#define SPA_STATIC_COUNTER_BYTES ((size_t)1 << 20)

enum { SPA_F32 = 0, SPA_F16 = 1, SPA_BF16 = 2 };
enum { SPA_SCORE_MAGNITUDE = 0, SPA_SCORE_WEIGHT = 1, SPA_SCORE_CLACT = 2 };
enum { SPA_SHIFT_NONE = 0, SPA_SHIFT_TOKEN_MEAN = 1, SPA_SHIFT_GIVEN = 2 };
enum { SPA_ACT_NONE = 0, SPA_ACT_RELU2 = 1 };
enum { SPA_META_BITMAP = 0, SPA_META_COMB = 1 };
enum { SPA_ENTRY_PRUNE = 0, SPA_ENTRY_DECODE = 1, SPA_ENTRY_PREFILL = 2 };

/* Pruning configuration.  m in {4, 8, 16, 32}; 1 <= n <= m; k % m == 0
 * (else SPA_ERR_INVALID).  The kernels are built for k % 16 == 0: a k of
 * whole m-blocks that is not returns SPA_ERR_UNSUPPORTED. */
typedef struct spa_prune_cfg {
  int32_t n;
  int32_t m;
  int32_t score;        /* SPA_SCORE_* */
  int32_t shift;        /* SPA_SHIFT_* */
  int32_t var_rescale;  /* 0, 1 (closed form) or 2 (running average) */
  int32_t act;          /* SPA_ACT_*: activation applied to the input first */
  /* var_rescale == 2 only: [device] [t] float32 per-token state in, and the
   * updated state out (must not alias); ignored otherwise. */
  const float* var_state;
  float* var_state_out;
} spa_prune_cfg;

/* A prepared linear layer.  Fields not needed by an entry point may be NULL:
 * one-token and float32 decode read wt, decode of 2..32 16-bit tokens and
 * prefill read w; chan_scale is needed for
 * SPA_SCORE_WEIGHT, row_sum whenever shift != SPA_SHIFT_NONE. */
typedef struct spa_weight {
  int32_t dtype;
  int32_t n_out;
  int32_t k;
  const void* w;            /* [device] [n_out][k], the layer's own layout        */
  const void* wt;           /* [device] [k][n_out], channel-major (from prepare)  */
  const float* chan_scale;  /* [device] [k], ||W[:,k]||_2^alpha (from prepare)    */
  const float* row_sum;     /* [device] [n_out], sum_k W[j,k] (from prepare)      */
} spa_weight;

/*
 * prepare_weight -- once per layer, off the timed path.
 * Writes wt = W^T ([k][n_out], so that channel k's weights are one
 * contiguous row and a pruned channel skips that whole row), chan_scale[c] =
 * float32((sum_j W[j,c]^2)^(alpha/2)) and row_sum[j] = float32(sum_c W[j,c]),
 * both sums formed in double-double arithmetic (WiSparse s2.1: the weight
 * norms can be computed ahead of time).  Any output pointer may be NULL to
 * skip it.  w: [device] [n_out][k].  Requires n_out >= 1, k >= 1,
 * 0 <= alpha <= 16.
 */
spa_status prepare_weight(const void* w, int32_t dtype, int32_t n_out, int32_t k, float alpha,
                          void* wt_out, float* chan_scale_out, float* row_sum_out, void* stream);

/*
 * prepare_amber -- once per layer, off the timed path: the Amber-Pruner
 * channel factor (activation sparsification guide s2.2.2), a drop-in
 * chan_scale for SPA_SCORE_WEIGHT:
 *   1. the 0.5th and 99.5th percentiles of all n_out*k weights (linear
 *      interpolation in float64 between the order statistics at floor and
 *      floor+1 of q/100 * (N-1)) bound the weights kept; the others are
 *      removed as outliers;
 *   2. the kept weights are standardised with their own mean and population
 *      standard deviation;
 *   3. chan_scale_out[c] = float32((sum over outputs j of the kept
 *      standardised W[j][c]^2)^(alpha/2)).
 * Order statistics by an exact radix select on the device; sums in
 * double-double arithmetic.  w: [device] [n_out][k]; chan_scale_out:
 * [device] [k]; workspace: [device] spa_amber_workspace_bytes() bytes (no
 * initial contents needed).  Requires n_out >= 1, k >= 1, 0 <= alpha <= 16.
 */
size_t spa_amber_workspace_bytes(void);
spa_status prepare_amber(const void* w, int32_t dtype, int32_t n_out, int32_t k, float alpha,
                         float* chan_scale_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Static per-token shift table (S-PTS, guide s3.1): calibration collects each
 * token's dynamic shift (the SPA_SHIFT_TOKEN_MEAN value) under a caller-given
 * token id; the table entry of an id is the mean of its collected shifts; at
 * run time a token's shift is its id's entry, passed as eta_in with
 * SPA_SHIFT_GIVEN.
 * spa_eta_calibrate -- x [device] [t][k] (k % 16 != 0: SPA_ERR_UNSUPPORTED),
 *   token_ids [device]
 *   [t] int32; adds each token's shift to sums[id] (float64) and 1 to
 *   counts[id] (uint32), both [device] [vocab] and zero-filled by the caller
 *   before the first batch.  Ids outside [0, vocab) are skipped.  The float64
 *   additions are atomic: their order, and so the last bits of a sum, may
 *   vary between runs.
 * spa_eta_table -- table[id] = float32(sums[id] / counts[id]), 0 when
 *   counts[id] == 0; all [device] [vocab].
 * spa_eta_lookup -- eta_out[i] = table[token_ids[i]] (0 for an id outside
 *   [0, vocab)); eta_out [device] [t] float32.
 */
spa_status spa_eta_calibrate(const void* x, int32_t dtype, int32_t t, int32_t k, const int32_t* token_ids,
                             int32_t vocab, double* sums, uint32_t* counts, void* stream);
spa_status spa_eta_table(const double* sums, const uint32_t* counts, int32_t vocab, float* table_out,
                         void* stream);
spa_status spa_eta_lookup(const float* table, int32_t vocab, const int32_t* token_ids, int32_t t, float* eta_out,
                          void* stream);

/*
 * prune_nm -- score, per-block top-n, pack (guide s2.1, s2.2, s3.1, s3.2).
 *  x          [device] [t][k]
 *  chan_scale [device] [k]   required iff cfg->score == SPA_SCORE_WEIGHT
 *  eta_in     [device] [t]   required iff cfg->shift == SPA_SHIFT_GIVEN
 *  vals_out   [device] [t][k*n/m] kept values of x_hat rounded to dtype
 *             (round-to-nearest-even), in ascending channel order
 *  idx_out    [device] [t][k*n/m] uint8 in-block position of each kept value
 *  eta_out    [device] [t] float32 or NULL
 *  nu_out     [device] [t] float32 or NULL (1.0 when cfg->var_rescale == 0)
 *  workspace  [device] spa_workspace_bytes(SPA_ENTRY_PRUNE, ...) bytes
 *             (only CLACT uses it; may be NULL otherwise)
 * Requires t >= 0 (t == 0 is a no-op), k >= m, k % m == 0.
 */
spa_status prune_nm(const void* x, int32_t dtype, int32_t t, int32_t k, const spa_prune_cfg* cfg,
                    const float* chan_scale, const float* eta_in, void* vals_out, uint8_t* idx_out,
                    float* eta_out, float* nu_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sparse_linear_decode -- the decode step, 1 <= t <= 32 tokens, float32
 * accumulation, y = nu * acc + eta * row_sum.
 *  - one token, and float32 (t <= 8): prune in registers, then stream
 *    only the rows of wt that some token of the call keeps (the
 *    memory-bound GEMV; guide s1.1 and s12.3: zero activations need not
 *    move, and bandwidth comes first).
 *  - 2..32 tokens of a 16-bit type: every token keeps its own n of each m
 *    channels, so their union covers most of wt (three quarters at two
 *    tokens of 8:16, nearly all from eight); a pruning pass writes the
 *    masked rows, and one pass over the row-major w on the matrix cores
 *    forms the product (per-token masks differ within a batch; WiSparse
 *    s5.1 separates small-batch from large-batch use).
 *  x        [device] [t][k]
 *  w        weight descriptor: wt required for one token and for float32
 *           (n_out % 8 == 0 for 16-bit dtypes, % 4 for float32); w->w
 *           required for 2..32 tokens of a 16-bit dtype
 *  eta_in   [device] [t], required iff cfg->shift == SPA_SHIFT_GIVEN
 *  y        [device] [t][n_out]
 *  idx_out  [device] [t][k*n/m] or NULL: the in-block positions the layer used
 *  nu_out   [device] [t] or NULL
 *  workspace [device] spa_workspace_bytes(SPA_ENTRY_DECODE, ...) bytes,
 *           zero-filled before its first use; each call leaves it reusable
 *           for later calls with the same sizes and configuration (zero it
 *           again before using it for other sizes).
 * Returns SPA_ERR_UNSUPPORTED for float32 with t > 8, for k % 16 != 0 and,
 * on the channel-major paths, for rows of wt that are not whole 16-byte
 * pieces (n_out % 8 != 0 in 16-bit dtypes, % 4 in float32).
 */
spa_status sparse_linear_decode(const void* x, int32_t t, const spa_weight* w, const spa_prune_cfg* cfg,
                                const float* eta_in, void* y, uint8_t* idx_out, float* nu_out,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * sparse_linear_decode_static -- sparse_linear_decode without a caller
 * workspace, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * call allocates nothing: its partial sums, variance sums, shift and split
 * counters live in one static device array per GPU of
 * SPA_STATIC_SCRATCH_BYTES (the first SPA_STATIC_COUNTER_BYTES are the
 * counters), which the library looks up once per GPU (with the current
 * device set to the stream's device) and clears there with a fill kernel on
 * `stream`.  Same kernels, arguments and results as sparse_linear_decode.
 *  - Returns SPA_ERR_SCRATCH, before any launch, when the call's decode
 *    workspace (spa_workspace_bytes(SPA_ENTRY_DECODE, ...)) exceeds
 *    SPA_STATIC_SCRATCH_BYTES - SPA_STATIC_COUNTER_BYTES or its column tiles
 *    need more than SPA_STATIC_COUNTER_BYTES / 4 counters.
 *  - Every call on a GPU shares that GPU's array and leaves its counters at
 *    zero; calls that overlap in time on one GPU (several streams, several
 *    threads) race and give undefined results.
 */
spa_status sparse_linear_decode_static(const void* x, int32_t t, const spa_weight* w, const spa_prune_cfg* cfg,
                                       const float* eta_in, void* y, uint8_t* idx_out, float* nu_out,
                                       void* stream);

/*
 * sparse_linear_prefill -- prompt-size batches, t >= 1 (16-bit dtypes):
 * a pruning pass packs the kept values, then an LDS-tiled matrix-core GEMM
 * with w ([n_out][k]) as the dense operand computes y.  2:4 runs on the
 * gfx950 sparse MFMA (smfmac), which skips the pruned half of the products
 * ("Accelerating Transformer training and inference with 2:4 sparsity and
 * Squared-ReLU" s2.1, s3.1); every other n:m runs dense MFMA on the
 * masked activations.
 *  Arguments as for sparse_linear_decode; w->w required, any n_out >= 1.
 *  workspace: spa_workspace_bytes(SPA_ENTRY_PREFILL, ...).
 *  SPA_ERR_UNSUPPORTED for float32, for k % 64 != 0 (whole 64-channel GEMM
 *  steps) and for k > 2^23 (8388608).
 */
spa_status sparse_linear_prefill(const void* x, int32_t t, const spa_weight* w, const spa_prune_cfg* cfg,
                                 const float* eta_in, void* y, uint8_t* idx_out, float* nu_out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * prepare_weight_fp8 -- FP8 copy of a weight for sparse_linear_prefill_fp8:
 * each row j of w ([n_out][k], 16-bit) becomes e4m3 codes (OCP FP8, 4
 * exponent and 3 mantissa bits, largest finite 448) of w[j][c] * (448 /
 * max_c |w[j][c]|), rounded to nearest even, with scale_out[j] = max |w[j]| /
 * 448 (0 and all-zero codes for an all-zero row).  One scale per row is the
 * granularity of the FP8 2:4 GEMM in "Accelerating Transformer training and
 * inference with 2:4 sparsity and Squared-ReLU" (s2.1, s3.1).
 *  w          [device] [n_out][k], SPA_F16 or SPA_BF16, 16-byte aligned
 *  codes_out  [device] [n_out][k] bytes, 16-byte aligned
 *  scale_out  [device] [n_out] float32
 * SPA_ERR_UNSUPPORTED for a float32 weight or k % 8 != 0.  Run once per
 * layer, off the hot path.
 */
spa_status prepare_weight_fp8(const void* w, int32_t dtype, int32_t n_out, int32_t k, uint8_t* codes_out,
                              float* scale_out, void* stream);

/*
 * sparse_linear_prefill_fp8 -- sparse_linear_prefill for 2:4 with both
 * operands in FP8 (the same paper, s2.1 and s3.1: the 2:4 product on FP8
 * tensors with per-row scales).  The pruning pass selects exactly as in
 * sparse_linear_prefill (idx_out, nu_out and the eta it uses are the same),
 * then stores each token's kept x - eta as e4m3 codes of (x - eta) * (448 /
 * a_i), a_i = max_c |x[i][c] - eta_i| over the whole row, with scale
 * sx_i = a_i / 448; the GEMM on v_smfmac_f32_32x32x64_fp8_fp8 accumulates
 * the code products in float32 and writes
 *   y[i][j] = nu_i * sx_i * sw_j * acc[i][j] + eta_i * row_sum[j].
 *  w        descriptor of the 16-bit weight: dtype, n_out, k, row_sum and
 *           chan_scale as for sparse_linear_prefill (w->w is not read)
 *  w_codes  [device] [n_out][k] from prepare_weight_fp8, 16-byte aligned
 *  w_scale  [device] [n_out] from prepare_weight_fp8
 *  Other arguments as for sparse_linear_prefill, same workspace size
 *  (spa_workspace_bytes(SPA_ENTRY_PREFILL, ...)).  SPA_ERR_UNSUPPORTED
 *  unless cfg is 2:4, and for k > 2^23.
 */
spa_status sparse_linear_prefill_fp8(const void* x, int32_t t, const spa_weight* w, const uint8_t* w_codes,
                                     const float* w_scale, const spa_prune_cfg* cfg, const float* eta_in, void* y,
                                     uint8_t* idx_out, float* nu_out, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Compact block metadata -- the in-block positions that prune_nm and the
 * linear calls return (uint8, ascending, n per m-block) to and from packed
 * per-block codes, for storing pruned activations (e.g. in a cache).
 *  SPA_META_COMB    ceil(log2 C(m, n)) bits per block (the guide's s2.1
 *                   table counts C(m, n) patterns per block; its s4.1 keeps a
 *                   2:4 block in 3 bits): the rank of the position set in
 *                   colexicographic order, sum_i C(c_i, i) over the
 *                   ascending positions c_1 < ... < c_n; 0 bits when n == m.
 *  SPA_META_BITMAP  m bits per block, bit j set when position j is kept.
 * Codes are laid end to end along a token row, block 0 in the lowest bits,
 * least significant bit first, in 32-bit words; each row starts on a new
 * word and its unused high bits are zero.
 *
 * spa_meta_row_bytes -- bytes of codes per token row: 4 * ceil((k/m) *
 *   bits per block / 32).  0 for invalid arguments as well.
 * spa_encode_meta -- idx [device] [t][k*n/m] uint8 -> codes [device]
 *   [t][row_bytes/4] uint32.  Positions that are not ascending or not below
 *   m give unspecified codes (never an access outside the buffers).
 * spa_decode_meta -- codes -> idx_out [device] [t][k*n/m].  A code that no
 *   n-subset has (a rank >= C(m, n), a mask without n set bits) gives
 *   unspecified positions below m.
 * Both require m in {4, 8, 16, 32}, 1 <= n <= m, k % m == 0, t >= 0 (0 is a
 * no-op), 16-byte aligned buffers.
 */
size_t spa_meta_row_bytes(int32_t k, int32_t n, int32_t m, int32_t format);
spa_status spa_encode_meta(const uint8_t* idx, int32_t t, int32_t k, int32_t n, int32_t m, int32_t format,
                           void* codes, void* stream);
spa_status spa_decode_meta(const void* codes, int32_t t, int32_t k, int32_t n, int32_t m, int32_t format,
                           uint8_t* idx_out, void* stream);

/*
 * sparse_ffn_relu2_prefill -- a squared-ReLU FFN whose activation is pruned
 * 2:4 on its way to the down-projection, with that activation never stored
 * dense ("Accelerating Transformer training and inference with 2:4 sparsity
 * and Squared-ReLU" s2.2, s3.1):
 *   u = x W_up^T (float32 accumulation, rounded to dtype);
 *   a = dtype(max(u, 0)^2);  keep 2 of every 4 by |a| (ties to the lower
 *   index);  y = (a * mask) W_down^T.
 * The up-projection's epilogue squares, prunes and packs its tile straight
 * into the 2:4 operand; the down-projection runs on the sparse MFMA.
 *  x       [device] [t][hidden]; up: w [ffn][hidden]; down: w [n_out][ffn]
 *          (only dtype, n_out, k and w of the descriptors are read)
 *  y       [device] [t][n_out]
 *  idx_out [device] [t][ffn/2] the kept positions of the activation, or NULL
 *  workspace [device] spa_ffn_workspace_bytes(t, ffn, dtype) bytes
 * Requires the same dtype for x, both weights and y, ffn % 4 == 0,
 * down.k == ffn, n_out >= 1 (else SPA_ERR_INVALID); SPA_ERR_UNSUPPORTED for
 * float32, for hidden or ffn not a multiple of 64 and for either above 2^23.
 * An activation value that ties exactly inside a block
 * keeps the lower index; because u comes from a float32-accumulating GEMM,
 * a near-tie can resolve differently from a float64 reference.
 */
size_t spa_ffn_workspace_bytes(int32_t t, int32_t ffn, int32_t dtype);
spa_status sparse_ffn_relu2_prefill(const void* x, int32_t t, const spa_weight* up, const spa_weight* down,
                                    void* y, uint8_t* idx_out, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * spa_prefill_layout -- where sparse_linear_prefill and
 * sparse_linear_prefill_fp8 keep the pruned operand inside their workspace
 * (for inspecting it after a call: tests, debugging; the calls do not need
 * it).  Byte offsets from the workspace start; a region the configuration
 * does not use has offset 0 and is not written.
 *  vals   2:4: per 64-channel step s and row r < t_pad, the step's 32 kept
 *         values in ascending channel order at ((s * t_pad) + r) * 32
 *         elements: dtype values, or on the FP8 path e4m3 codes (one byte
 *         each, 32 bytes per row and step).  Other n:m: the masked rows
 *         [t][k] (dtype, zeros at pruned channels).
 *  meta   2:4 only: per step and row four uint16 words at ((s * t_pad) + r)
 *         * 4, word q holding the 16 channels 16q..16q+15 of the step as
 *         four nibbles (block b in bits 4b..4b+3: lo | hi << 2, the two kept
 *         in-block positions).
 *  eta    [t] float32, the shift the call used.
 *  scale  FP8 path only: [t] float32, each token's scale max|kept x_hat| / 448.
 *  t_pad  rows per step of the 2:4 layout (t rounded up to 256); t otherwise.
 *  bytes  the workspace size (spa_workspace_bytes(SPA_ENTRY_PREFILL, ...)).
 * SPA_ERR_INVALID for arguments spa_workspace_bytes rejects, or a NULL out.
 */
typedef struct spa_operand_layout {
  size_t vals, meta, eta, scale;
  int32_t t_pad;
  size_t bytes;
} spa_operand_layout;
spa_status spa_prefill_layout(int32_t t, int32_t k, int32_t dtype, const spa_prune_cfg* cfg,
                              spa_operand_layout* out);

/* Workspace bytes an entry point needs for these sizes (0 if none); 0 for
 * invalid arguments as well. */
size_t spa_workspace_bytes(int32_t entry, int32_t t, int32_t k, int32_t n_out, int32_t dtype,
                           const spa_prune_cfg* cfg);

/* Static, NUL-terminated description of a status code. */
const char* spa_status_str(spa_status s);

#ifdef __cplusplus
}
#endif

#endif /* SPA_H_ */

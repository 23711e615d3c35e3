"""CPU oracle for input-adaptive N:M activation pruning fused with a linear layer.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the package's
smoke check and the benchmark's CPU-baseline leg may import this module.  It
shares no code, table or constant with the HIP library and never imports it.

Plain, slow, obviously-correct numpy.  The mask pipeline runs in float32, one
IEEE-rounded elementwise operation at a time (numpy never fuses a multiply
and an add); sums whose order would matter are taken exactly with
``math.fsum`` and rounded once.  The output ``y`` and the variance factor run
in float64.

Sources (page titles; sections as numbered on each page):

* [Guide]   "Activation sparsification: a dynamic pruning method for efficient
            LLM inference" -- s2.1 N:M patterns table, s2.2.1 magnitude pruning
            (ACT), s2.2.3 cosine-loss activation score (CLACT), s3.1 dynamic
            per-token shift (D-PTS / S-PTS), s3.2 variance correction (VAR),
            s6.1 prototype N:M operator.
* [WiSparse] "LLM inference optimisation: WiSparse activation sparsification
            explained" -- s2.1, equation (4): weight-aware channel score.
* [SqReLU]  "Accelerating Transformer training and inference with 2:4
            sparsity and Squared-ReLU" -- s2.2: the activation max(0, x)^2;
            s3.1: one kernel applies it, prunes 2:4 and packs; s3.3:
            non-zeros stored contiguously with a mask.

Readings taken where the pages are silent or disagree (each is listed in the
design notes as well):

* Ties at the top-N boundary: exactly N are kept per block and, among equal
  scores, the lower in-block index wins.  (The magnitude code in [Guide]
  s2.2.1 keeps every value >= the N-th largest, so it keeps more than N on
  ties; the prototype in s6.1 leaves the tie order to ``topk``.)
* What is scored under a shift: |x - eta| (the shifted value is pruned and
  kept).
* The weight norm of channel k is taken over the outputs: for y = x W^T with
  W[n_out, k], it is the 2-norm of column k of W.
* Amber-Pruner factor ([Guide] s2.2.2): the 0.5th and 99.5th percentiles of
  all weights of the matrix (linear interpolation between order statistics,
  in float64) bound the weights kept; the kept weights are standardised with
  their own mean and population standard deviation; f_k is the 2-norm over
  the outputs of channel k's standardised kept weights, to the power alpha.
  The standard deviation scales every f_k alike, so it cannot change a mask.
* f_k = ||W[:,k]||_2^alpha is formed once from the exact sum of squares,
  raised to alpha/2 in float64 and rounded to float32.
* eta (D-PTS) = float32(float64(exact row sum) / K).
* S-PTS table ([Guide] s3.1): calibration collects each token's D-PTS shift
  under the caller's token id; the table entry of an id is the mean of its
  collected shifts (exact sum, divided in float64, rounded to float32), 0
  for an id never seen; at run time a token takes its id's entry.
* CLACT: the column energy runs over the tokens of the call, squares and
  adds rounded in float32 with tokens in ascending order, then a correctly
  rounded float32 square root.  The per-row factor 1/||x_i|| is a positive
  constant of the row and cannot change any in-block ranking, so the score
  is |x_ik - eta_i| * c_k.
* VAR: the closed form of [Guide] s3.2 per token, population variances in
  float64 over all K positions; a zero denominator gives nu = 1.
* VAR, running-average form (the implementation note of the same section):
  per token slot a state r, updated as r <- 0.9 r + 0.1 Var[x_hat]; then
  nu = sqrt(r / (Var[x_hat * m] + 1e-6)).  The listing divides by the dense
  variance, which would make nu ~ 1; the masked variance of the closed form
  is taken instead.  State and arithmetic in float64, stored as float32.
* The dense term of (x_sparse + eta) W^T is split as
  (x_hat * m) W^T + eta * (W 1): only kept rows of W^T are read.
* Squared ReLU as the input transform: max(0, u)^2 in float32, rounded to
  the storage dtype -- what a separate elementwise pass would store; the
  fused kernel must see the same input.
* Compact block metadata ([Guide] s2.1 table, s4.1: 3 bits per 2:4 block):
  a block's kept positions as one code of ceil(log2 C(m, n)) bits -- the
  rank of the position set in colexicographic order (the combinatorial
  number system: sum over the ascending positions c_1 < ... < c_n of
  C(c_i, i)) -- or as an m-bit mask (bit j = position j kept).  Codes are
  laid end to end, block 0 in the lowest bits, least significant bit
  first, in 32-bit words; each row starts on a fresh word.
* FP8 2:4 prefill ([SqReLU] s3.1: FP8 with row scales; s5.3: sparsify,
  then quantise): e4m3 in the OCP form (bias 7, largest 448, no infinity),
  rounded to nearest even; activation rows scaled by 448 / max|x_hat| of the
  row, weight rows by 448 / max|w| of the row, both float32; y takes the
  float64 product of the codes times both scales.
* Packed values are the float32 shifted values rounded to the storage dtype
  (round-to-nearest-even); the index metadata is one uint8 in-block position
  per kept value, ascending.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")


# ----------------------------------------------------------------------------
# Storage-dtype rounding
# ----------------------------------------------------------------------------

def round_to_dtype(v: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (round-to-nearest-even).

    Returns float32 values exactly representable in ``dtype``.  bfloat16 is
    the upper 16 bits of an IEEE binary32; rounding to nearest-even adds
    0x7FFF plus the lowest kept bit before truncating (finite inputs only).
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    if dtype == "f32":
        return v.copy()
    if dtype == "f16":
        return v.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        u = v.view(np.uint32).astype(np.uint64)
        lsb = (u >> np.uint64(16)) & np.uint64(1)
        r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
        return r.astype(np.uint32).view(np.float32)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Weight-side precomputation (off the timed path)
# ----------------------------------------------------------------------------

def channel_factor(w: np.ndarray, alpha: float) -> np.ndarray:
    """f_k = ||W[:,k]||_2 ** alpha as float32  ([WiSparse] s2.1, eq. (4)).

    ``w`` is [n_out, k] (float32 values of the stored weight).  The sum of
    squares is exact (``math.fsum``; each square of a float32 is exact in
    float64), rounded once to float64; the power is taken as
    ``sumsq ** (alpha / 2)`` in float64 and rounded to float32.
    """
    w64 = np.asarray(w, dtype=np.float64)
    sq = w64 * w64                      # exact: 24x24-bit products fit in 53 bits
    k = w64.shape[1]
    f = np.empty(k, dtype=np.float32)
    for c in range(k):
        sumsq = math.fsum(sq[:, c].tolist())
        f[c] = np.float32(sumsq ** (alpha / 2.0))
    return f


def percentile_linear(v_sorted: np.ndarray, q: float) -> float:
    """The q-th percentile (0..100) of sorted values: interpolate between the
    order statistics at floor and ceil of q/100 * (N - 1), in float64."""
    n = v_sorted.size
    pos = q / 100.0 * (n - 1)
    i = int(math.floor(pos))
    g = pos - i
    a = float(v_sorted[i])
    b = float(v_sorted[min(i + 1, n - 1)])
    return a + (b - a) * g


def amber_factor(w: np.ndarray, alpha: float = 1.0, q_lo: float = 0.5, q_hi: float = 99.5, cols=None) -> np.ndarray:
    """Amber-Pruner channel factor ([Guide] s2.2.2), float32 [k].

    1. keep the weights between the q_lo-th and q_hi-th percentiles of the
       whole matrix (outliers are removed);
    2. standardise the kept weights: z = (w - mean) / std (their own mean and
       population standard deviation);
    3. f_k = (sum over outputs j of z_jk^2, kept weights only) ** (alpha / 2).
    Differences and squares are float64, their sums exact (math.fsum) and
    rounded once; the ratio and the power are float64, the result float32.
    ``cols`` restricts step 3 to those channels (the result holds only them).
    """
    w64 = np.asarray(w, dtype=np.float64)
    v = np.sort(w64.ravel())
    lo, hi = percentile_linear(v, q_lo), percentile_linear(v, q_hi)
    kept = (w64 >= lo) & (w64 <= hi)
    vals = w64[kept]
    cnt = vals.size
    mean = math.fsum(vals.tolist()) / cnt
    dev = vals - mean
    var = math.fsum((dev * dev).tolist()) / cnt
    cols = range(w64.shape[1]) if cols is None else list(cols)
    f = np.empty(len(cols), dtype=np.float32)
    for out_i, c in enumerate(cols):
        col = w64[kept[:, c], c]
        d = col - mean
        ss = math.fsum((d * d).tolist()) / var if var > 0 else 0.0
        f[out_i] = np.float32(ss ** (alpha / 2.0))
    return f


def row_sum(w: np.ndarray) -> np.ndarray:
    """s_j = sum_k W[j,k], exact then rounded to float64 (the W 1 of the shift term)."""
    w64 = np.asarray(w, dtype=np.float64)
    return np.array([math.fsum(r.tolist()) for r in w64], dtype=np.float64)


# ----------------------------------------------------------------------------
# Per-token steps ([Guide] s2.2, s3.1, s3.2; [WiSparse] s2.1)
# ----------------------------------------------------------------------------

def squared_relu(u: np.ndarray, dtype: str) -> np.ndarray:
    """x = max(0, u)^2 ([SqReLU] s2.2), as the layer input the pruning sees.

    The square is one float32 multiply (exact when u is a 16-bit value) and
    the result is rounded to the storage dtype, to nearest even.
    """
    u = np.asarray(u, dtype=np.float32)
    r = np.where(u > 0, u, np.float32(0.0)).astype(np.float32)
    return round_to_dtype(r * r, dtype)


def token_mean(x: np.ndarray) -> np.ndarray:
    """D-PTS shift eta_i = mean over channels of x_i  ([Guide] s3.1).

    float32(float64(exact sum) / K).
    """
    x64 = np.asarray(x, dtype=np.float64)
    k = x64.shape[1]
    return np.array([np.float32(math.fsum(r.tolist()) / k) for r in x64], dtype=np.float32)


def eta_table(batches, vocab: int) -> np.ndarray:
    """S-PTS table from calibration batches ([Guide] s3.1), float32 [vocab].

    ``batches``: iterable of (x [t, k] float32 values, token_ids [t]).  Each
    token's D-PTS shift (``token_mean``) is collected under its id; entry id
    is float32(float64(exact sum of its shifts) / count), 0 when unseen.
    """
    buf = [[] for _ in range(vocab)]
    for x, ids in batches:
        eta = token_mean(x)
        for e, i in zip(eta.tolist(), np.asarray(ids).tolist()):
            buf[int(i)].append(float(e))
    return np.array([np.float32(math.fsum(b) / len(b)) if b else np.float32(0.0) for b in buf], dtype=np.float32)


def eta_lookup(table: np.ndarray, ids) -> np.ndarray:
    """A token's static shift: its id's table entry; 0 for an id outside the table."""
    table = np.asarray(table, dtype=np.float32)
    ids = np.asarray(ids, dtype=np.int64)
    ok = (ids >= 0) & (ids < table.size)
    return np.where(ok, table[np.clip(ids, 0, table.size - 1)], np.float32(0.0)).astype(np.float32)


def shift(x: np.ndarray, eta: np.ndarray) -> np.ndarray:
    """x_hat = x - eta, one float32 subtraction per element ([Guide] s3.1)."""
    return np.asarray(x, dtype=np.float32) - np.asarray(eta, dtype=np.float32)[:, None]


def clact_colnorm(xhat: np.ndarray) -> np.ndarray:
    """CLACT column energy c_k = sqrt(sum_p xhat_pk^2)  ([Guide] s2.2.3).

    Tokens in ascending order; every square and every add rounded to float32;
    correctly rounded float32 square root.
    """
    xhat = np.asarray(xhat, dtype=np.float32)
    acc = np.zeros(xhat.shape[1], dtype=np.float32)
    for p in range(xhat.shape[0]):
        sq = xhat[p] * xhat[p]
        acc = acc + sq
    return np.sqrt(acc)


def scores(xhat: np.ndarray, f: Optional[np.ndarray]) -> np.ndarray:
    """score_ik = |xhat_ik| * f_k, one float32 multiply ([Guide] s2.2.1, [WiSparse] eq. (4)).

    ``f`` None means the magnitude criterion (f = 1).
    """
    a = np.abs(np.asarray(xhat, dtype=np.float32))
    if f is None:
        return a
    return a * np.asarray(f, dtype=np.float32)[None, :]


def topn_mask(score: np.ndarray, n: int, m: int) -> np.ndarray:
    """Keep the top-n of every m consecutive channels ([Guide] s2.1).

    Position k of a block is kept iff fewer than n positions j of the same
    block beat it, where j beats k when score_j > score_k, or the scores are
    equal and j < k.  Exactly n are kept per block.
    """
    t, k = score.shape
    s = np.asarray(score, dtype=np.float32).reshape(t, k // m, m)
    sj = s[:, :, :, None]          # candidate beater j on axis 2
    sk = s[:, :, None, :]          # position k on axis 3
    j_idx = np.arange(m)[:, None]
    k_idx = np.arange(m)[None, :]
    beats = (sj > sk) | ((sj == sk) & (j_idx < k_idx))
    rank = beats.sum(axis=2)
    return (rank < n).reshape(t, k)


def pack(xhat: np.ndarray, keep: np.ndarray, n: int, m: int, dtype: str):
    """Packed kept values plus uint8 in-block positions, ascending ([SqReLU] s3.3).

    Returns ``(vals, idx)``: ``vals`` [t, k*n/m] float32 holding the values of
    ``dtype`` (round-to-nearest-even of the float32 x_hat); ``idx`` [t, k*n/m]
    uint8.
    """
    t, k = xhat.shape
    pos = np.broadcast_to(np.tile(np.arange(m, dtype=np.uint8), k // m), (t, k))
    idx = pos[keep].reshape(t, k // m * n)
    vals = round_to_dtype(xhat, dtype)[keep].reshape(t, k // m * n)
    return vals, idx


def var_factor(xhat: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """nu_i = sqrt(Var[x_hat_i] / Var[x_hat_i * m_i])  ([Guide] s3.2), float64 -> float32.

    Population variances over all K positions (the 1/K vs 1/(K-1) choice
    cancels in the ratio).  A zero denominator gives nu = 1.
    """
    xh = np.asarray(xhat, dtype=np.float64)
    xm = xh * keep
    num = xh.var(axis=1)
    den = xm.var(axis=1)
    nu = np.ones(xh.shape[0], dtype=np.float64)
    ok = den > 0
    nu[ok] = np.sqrt(num[ok] / den[ok])
    return nu.astype(np.float32)


def var_factor_ema(xhat: np.ndarray, keep: np.ndarray, r_in, decay: float = 0.9, gain: float = 0.1,
                   eps: float = 1e-6):
    """Running-average VAR ([Guide] s3.2): returns (nu, r_out), both float32 [t].

    r_out_i = decay * r_in_i + gain * Var[x_hat_i] (0.9 and 0.1 as printed);
    nu_i = sqrt(r_out_i / (Var[x_hat_i * m_i] + eps)).  Population variances,
    float64 throughout.
    """
    xh = np.asarray(xhat, dtype=np.float64)
    num = xh.var(axis=1)
    den = (xh * keep).var(axis=1)
    r = decay * np.asarray(r_in, dtype=np.float64) + gain * num
    nu = np.sqrt(r / (den + eps))
    return nu.astype(np.float32), r.astype(np.float32)


# ----------------------------------------------------------------------------
# The whole pruning step and the linear layer
# ----------------------------------------------------------------------------

def prune(x, dtype: str, n: int, m: int, score: str = "magnitude", f=None, shift_mode: str = "none",
          eta_in=None, var_rescale=False, act: str = "none", var_state=None) -> dict:
    """(Activation) -> score -> per-block top-n -> pack -> (nu), for X[t, k] given as float32 values.

    ``act``: "none" | "relu2" (``x`` is then the pre-activation u, and the
    layer input is ``squared_relu(u)``).
    ``score``: "magnitude" | "weight" (needs ``f``) | "clact".
    ``shift_mode``: "none" | "token_mean" (D-PTS) | "given" (S-PTS, ``eta_in``).
    """
    x = np.asarray(x, dtype=np.float32)
    if act == "relu2":
        x = squared_relu(x, dtype)
    elif act != "none":
        raise ValueError(act)
    t, k = x.shape
    if not (1 <= n <= m) or k % m:
        raise ValueError("need 1 <= n <= m and m | k")
    if shift_mode == "none":
        eta = np.zeros(t, dtype=np.float32)
    elif shift_mode == "token_mean":
        eta = token_mean(x)
    elif shift_mode == "given":
        eta = np.asarray(eta_in, dtype=np.float32).copy()
    else:
        raise ValueError(shift_mode)
    xhat = shift(x, eta)
    if score == "magnitude":
        factor = None
    elif score == "weight":
        factor = np.asarray(f, dtype=np.float32)
    elif score == "clact":
        factor = clact_colnorm(xhat)
    else:
        raise ValueError(score)
    sc = scores(xhat, factor)
    keep = topn_mask(sc, n, m)
    vals, idx = pack(xhat, keep, n, m, dtype)
    out = dict(eta=eta, xhat=xhat, factor=factor, score=sc, keep=keep, vals=vals, idx=idx)
    if var_rescale == 2:                     # running-average form, state var_state [t]
        out["nu"], out["var_state"] = var_factor_ema(xhat, keep, var_state)
    else:
        out["nu"] = var_factor(xhat, keep) if var_rescale else np.ones(t, dtype=np.float32)
    return out


def linear(pr: dict, w, s=None) -> np.ndarray:
    """y_i = nu_i * (x_hat_i * m_i) W^T + eta_i * (W 1), float64  ([Guide] s3.1, s3.2).

    ``w`` [n_out, k] float32 values; ``s`` the exact row sums (computed when None).
    """
    w64 = np.asarray(w, dtype=np.float64)
    if s is None:
        s = row_sum(w)
    xs = pr["xhat"].astype(np.float64) * pr["keep"]
    y = xs @ w64.T
    y = pr["nu"].astype(np.float64)[:, None] * y
    return y + pr["eta"].astype(np.float64)[:, None] * np.asarray(s, dtype=np.float64)[None, :]


def linear_pages_form(pr: dict, w) -> np.ndarray:
    """The shifted output exactly as [Guide] s3.1 writes it: (x_sparse + eta) W^T (no nu)."""
    w64 = np.asarray(w, dtype=np.float64)
    xs = pr["xhat"].astype(np.float64) * pr["keep"] + pr["eta"].astype(np.float64)[:, None]
    return xs @ w64.T


# ----------------------------------------------------------------------------
# Compact block metadata ([Guide] s2.1 table, s4.1)
# ----------------------------------------------------------------------------

META_FORMATS = ("bitmap", "comb")


def meta_width(n: int, m: int, fmt: str) -> int:
    """Bits per m-block: m for the mask, ceil(log2 C(m, n)) for the combinatorial code."""
    if fmt == "bitmap":
        return m
    if fmt == "comb":
        count = math.comb(m, n)
        return (count - 1).bit_length()            # ceil(log2 count); 0 when only one subset exists
    raise ValueError(fmt)


def meta_row_words(k: int, n: int, m: int, fmt: str) -> int:
    """32-bit words per token row of codes."""
    return ((k // m) * meta_width(n, m, fmt) + 31) // 32


def comb_rank(positions) -> int:
    """Colexicographic rank of an ascending position set: sum_i C(c_i, i), i = 1..n."""
    return sum(math.comb(int(c), i + 1) for i, c in enumerate(positions))


def comb_unrank(r: int, n: int, m: int) -> list:
    """The ascending n-subset of range(m) with colexicographic rank r (greedy, largest first)."""
    out = []
    c = m
    for i in range(n, 0, -1):
        c -= 1
        while math.comb(c, i) > r:
            c -= 1
        out.append(c)
        r -= math.comb(c, i)
    return out[::-1]


def encode_meta(idx: np.ndarray, n: int, m: int, fmt: str) -> np.ndarray:
    """uint8 in-block positions [t, k*n/m] -> uint32 codes [t, row_words]."""
    idx = np.asarray(idx, dtype=np.int64)
    t = idx.shape[0]
    nb = idx.shape[1] // n
    w = meta_width(n, m, fmt)
    words = meta_row_words(nb * m, n, m, fmt)
    out = np.zeros((t, words), dtype=np.uint32)
    for r in range(t):
        acc = 0
        for b in range(nb):
            pos = idx[r, b * n:(b + 1) * n]
            code = comb_rank(pos) if fmt == "comb" else sum(1 << int(c) for c in pos)
            acc |= code << (b * w)
        for j in range(words):
            out[r, j] = (acc >> (32 * j)) & 0xFFFFFFFF
    return out


def decode_meta(codes: np.ndarray, k: int, n: int, m: int, fmt: str) -> np.ndarray:
    """uint32 codes [t, row_words] -> uint8 in-block positions [t, k*n/m]."""
    codes = np.asarray(codes, dtype=np.uint32)
    t = codes.shape[0]
    nb = k // m
    w = meta_width(n, m, fmt)
    out = np.zeros((t, nb * n), dtype=np.uint8)
    for r in range(t):
        acc = 0
        for j in range(codes.shape[1]):
            acc |= int(codes[r, j]) << (32 * j)
        for b in range(nb):
            code = (acc >> (b * w)) & ((1 << w) - 1)
            if fmt == "comb":
                pos = comb_unrank(code, n, m)
            else:
                pos = [c for c in range(m) if (code >> c) & 1]
            out[r, b * n:(b + 1) * n] = pos
    return out


def ffn_relu2(x, w_up, w_down, dtype: str) -> dict:
    """Squared-ReLU FFN with its activation pruned 2:4 ([SqReLU] s2.2, s3.1).

    u = the up-projection x W_up^T as a float32-accumulating GEMM stores it:
    the exact sum rounded to float32, then to ``dtype``; the activation
    squared_relu(u) is pruned 2:4 by magnitude (no shift); y = the
    down-projection of the pruned activation, float64.
    Returns the prune record (``u`` included) with ``y``.
    """
    x64 = np.asarray(x, dtype=np.float64)
    u = round_to_dtype((x64 @ np.asarray(w_up, dtype=np.float64).T).astype(np.float32), dtype)
    pr = prune(u, dtype, 2, 4, act="relu2")
    pr["u"] = u
    pr["y"] = linear(pr, w_down, s=np.zeros(np.asarray(w_down).shape[0]))
    return pr


# ----------------------------------------------------------------------------
# FP8 (e4m3) 2:4 prefill ([SqReLU] s3.1, s5.3)
# ----------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Value of an OCP e4m3 byte: sign, 4 exponent bits (bias 7), 3 mantissa bits;
    exponent 0 is subnormal; 0x7F / 0xFF are NaN; no infinity."""
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """float32 values -> e4m3 codes (uint8), nearest value, ties to the even code.

    The sign bit is the operand's, also when the result is zero: the format has
    both zeros (0x00, 0x80) and IEEE rounding keeps the sign of a zero result.

    |v| is assumed <= 464 (the scaled operands stay within 448 up to one
    float32 rounding); larger inputs are outside the format."""
    table = [(e4m3_value(c), c) for c in range(128) if c != 0x7F]   # non-negative values, ascending
    vals = np.array([t[0] for t in table])
    codes = np.array([t[1] for t in table], dtype=np.uint8)
    x = np.asarray(v, dtype=np.float64).ravel()
    a = np.abs(x)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, vals.size - 1)
    lo = np.clip(hi - 1, 0, vals.size - 1)
    dl, dh = a - vals[lo], vals[hi] - a
    pick_hi = (dh < dl) | ((dh == dl) & (codes[hi] % 2 == 0) & (hi != lo))
    c = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    c = np.where(a == vals[hi], codes[hi], c).astype(np.uint8)
    neg = np.signbit(x)
    return (c | np.where(neg, 0x80, 0).astype(np.uint8)).reshape(np.shape(v))


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    lut = np.array([e4m3_value(c) for c in range(256)])
    return lut[np.asarray(codes, dtype=np.int64)]


def fp8_rows(v: np.ndarray):
    """Per-row scale s = float32(max|v| / 448) and codes e4m3(float32(v * float32(448 / max|v|)));
    a zero row gets s = 0 and zero codes."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.abs(v).max(axis=1).astype(np.float32)
    ok = amax > 0
    inv = np.where(ok, np.float32(448.0) / np.where(ok, amax, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    scale = np.where(ok, amax / np.float32(448.0), np.float32(0.0)).astype(np.float32)
    return e4m3_round((v * inv[:, None]).astype(np.float32)), scale


def prefill_fp8(x, w, dtype: str, score: str = "magnitude", f=None, shift_mode: str = "none", eta_in=None,
                var_rescale=False, s=None, act: str = "none", var_state=None) -> dict:
    """2:4 prefill with FP8 operands: the mask of ``prune`` (on the 16-bit input),
    then the sparsified x_hat quantised per token ([SqReLU] s5.3: sparsify
    first, then quantise -- the token's scale is the largest kept |x_hat|),
    W quantised per output row;
    y_ij = nu_i * sx_i * sw_j * sum_k qx_ik qw_jk + eta_i * s_j (float64)."""
    pr = prune(x, dtype, 2, 4, score=score, f=f, shift_mode=shift_mode, eta_in=eta_in, var_rescale=var_rescale,
               act=act, var_state=var_state)
    xs = np.where(pr["keep"], pr["xhat"], np.float32(0.0)).astype(np.float32)
    qx, sx = fp8_rows(xs)
    qx = np.where(pr["keep"], qx, 0).astype(np.uint8)
    qw, sw = fp8_rows(w)
    if s is None:
        s = row_sum(w)
    acc = e4m3_decode(qx) @ e4m3_decode(qw).T
    y = pr["nu"].astype(np.float64)[:, None] * (sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :] * acc)
    pr.update(qx=qx, sx=sx, qw=qw, sw=sw, xs=xs)
    pr["y"] = y + pr["eta"].astype(np.float64)[:, None] * np.asarray(s, dtype=np.float64)[None, :]
    return pr


def rowwise_error(y_test: np.ndarray, y_ref: np.ndarray) -> float:
    """max_i ( max_j |y_test - y_ref| / max_j |y_ref| ): the row-normwise relative error."""
    y_test = np.asarray(y_test, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y_ref.size == 0:
        return 0.0
    num = np.abs(y_test - y_ref).max(axis=1)
    den = np.abs(y_ref).max(axis=1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())


TOLERANCE = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}

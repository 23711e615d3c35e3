"""Planted-mistake check of the oracle's pins (CPU only).

Each case swaps one oracle function for a plausible wrong variant (on the
CPU, in this process only) and asserts that at least one pin in
``test_oracle_pins`` then fails.  This shows the pins are tight enough to
catch that class of slip.
"""
import math

import numpy as np
import pytest

from oracle import nm_oracle as O
import test_oracle_pins as P


def _tie_high(score, n, m):
    t, k = score.shape
    s = score.reshape(t, k // m, m)
    sj, sk = s[:, :, :, None], s[:, :, None, :]
    j, kk = np.arange(m)[:, None], np.arange(m)[None, :]
    beats = (sj > sk) | ((sj == sk) & (j > kk))          # wrong: higher index wins
    return (beats.sum(axis=2) < n).reshape(t, k)


def _ge_threshold(score, n, m):                          # keeps > n on ties
    t, k = score.shape
    b = score.reshape(t, k // m, m)
    thr = -np.sort(-b, axis=-1)[..., n - 1:n]
    return (b >= thr).reshape(t, k)


def _shift_plus(x, eta):
    return np.asarray(x, np.float32) + np.asarray(eta, np.float32)[:, None]


def _linear_no_eta(pr, w, s=None):
    w64 = np.asarray(w, np.float64)
    xs = pr["xhat"].astype(np.float64) * pr["keep"]
    return pr["nu"].astype(np.float64)[:, None] * (xs @ w64.T)


def _factor_rows(w, alpha):                              # transposed operand: norm of rows
    f = _orig_factor(np.asarray(w).T.copy(), alpha)
    return np.resize(f, np.asarray(w).shape[1]).astype(np.float32)


def _var_inverted(xhat, keep):
    nu = _orig_var(xhat, keep)
    return (1.0 / nu).astype(np.float32)


def _clact_abs(xhat):
    return np.abs(np.asarray(xhat, np.float32)).sum(axis=0).astype(np.float32)


def _mean_wrong_div(x):
    x64 = np.asarray(x, np.float64)
    return np.float32(x64.sum(axis=1) / (x64.shape[1] - 1))


def _bf16_truncate(v, dtype):
    v = np.ascontiguousarray(v, np.float32)
    if dtype == "bf16":
        return (v.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    return _orig_round(v, dtype)


def _relu2_abs(u, dtype):                                # squares negative inputs too
    u = np.asarray(u, np.float32)
    return _orig_round(u * u, dtype)


def _relu2_unrounded(u, dtype):                          # keeps the float32 square
    u = np.asarray(u, np.float32)
    r = np.where(u > 0, u, np.float32(0)).astype(np.float32)
    return r * r


def _relu_only(u, dtype):                                # forgets the square
    u = np.asarray(u, np.float32)
    return _orig_round(np.where(u > 0, u, np.float32(0)).astype(np.float32), dtype)


def _lex_rank(positions):                                # lexicographic instead of colex order
    m = 32
    n = len(positions)
    r, prev = 0, -1
    for i, c in enumerate(positions):
        for v in range(prev + 1, int(c)):
            r += math.comb(m - 1 - v, n - 1 - i)
        prev = int(c)
    return r


def _width_floor(n, m, fmt):                             # floor instead of ceil of log2
    if fmt == "comb":
        return max(0, math.comb(m, n).bit_length() - 1)
    return m


def _amber_no_removal(w, alpha=1.0, q_lo=0.5, q_hi=99.5):   # keeps the outliers
    return _orig_amber(w, alpha, 0.0, 100.0)


def _amber_raw_norm(w, alpha=1.0, q_lo=0.5, q_hi=99.5):      # skips the standardisation
    w64 = np.asarray(w, np.float64)
    v = np.sort(w64.ravel())
    lo, hi = O.percentile_linear(v, q_lo), O.percentile_linear(v, q_hi)
    kept = (w64 >= lo) & (w64 <= hi)
    ss = np.where(kept, w64 * w64, 0.0).sum(axis=0)
    return (ss ** (alpha / 2)).astype(np.float32)


def _eta_table_last(batches, vocab):                     # keeps the last shift, not the mean
    tab = np.zeros(vocab, np.float32)
    for x, ids in batches:
        for e, i in zip(O.token_mean(x).tolist(), np.asarray(ids).tolist()):
            tab[int(i)] = e
    return tab


def _ema_dense_denominator(xhat, keep, r_in, decay=0.9, gain=0.1, eps=1e-6):   # divides by the dense variance
    xh = np.asarray(xhat, np.float64)
    num = xh.var(axis=1)
    r = decay * np.asarray(r_in, np.float64) + gain * num
    return np.sqrt(r / (num + eps)).astype(np.float32), r.astype(np.float32)


def _e4m3_truncate(v):                                   # rounds toward zero
    table = [(O.e4m3_value(c), c) for c in range(0x7F)]
    out = []
    for x in np.asarray(v, np.float64).ravel().tolist():
        c = max(c for val, c in table if val <= abs(x))
        out.append(c | (0x80 if x < 0 and c else 0))
    return np.array(out, np.uint8).reshape(np.shape(v))


def _fp8_column_scales(v):                               # scales over the wrong axis
    q, sc = _orig_fp8_rows(np.asarray(v, np.float32).T.copy())
    return q.T.copy(), sc


def _fp8_inverted_scale(v):                              # stores 448 / max instead of max / 448
    q, sc = _orig_fp8_rows(v)
    return q, np.where(sc > 0, np.float32(1.0) / np.where(sc > 0, sc, 1), 0).astype(np.float32)


def _fp8_whole_row_scale(x, w, dtype, score="magnitude", f=None, shift_mode="none", eta_in=None, var_rescale=False,
                         s=None, act="none", var_state=None):   # token scale over the whole row, pruned entries too
    pr = O.prune(x, dtype, 2, 4, score=score, f=f, shift_mode=shift_mode, eta_in=eta_in, var_rescale=var_rescale,
                 act=act, var_state=var_state)
    qx, sx = O.fp8_rows(pr["xhat"])
    qx = np.where(pr["keep"], qx, 0).astype(np.uint8)
    qw, sw = O.fp8_rows(w)
    s = O.row_sum(w) if s is None else s
    acc = O.e4m3_decode(qx) @ O.e4m3_decode(qw).T
    y = pr["nu"].astype(np.float64)[:, None] * (sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :] * acc)
    pr.update(qx=qx, sx=sx, qw=qw, sw=sw)
    pr["y"] = y + pr["eta"].astype(np.float64)[:, None] * np.asarray(s, np.float64)[None, :]
    return pr


_orig_fp8_rows = O.fp8_rows
_orig_factor = O.channel_factor
_orig_amber = O.amber_factor
_orig_var = O.var_factor
_orig_round = O.round_to_dtype

PINS = [name for name in dir(P) if name.startswith("test_")]

MUTANTS = {
    "tie_to_higher_index": ("topn_mask", _tie_high),
    "threshold_keeps_ties": ("topn_mask", _ge_threshold),
    "shift_sign": ("shift", _shift_plus),
    "drop_shift_term": ("linear", _linear_no_eta),
    "factor_transposed": ("channel_factor", _factor_rows),
    "nu_inverted": ("var_factor", _var_inverted),
    "clact_no_square": ("clact_colnorm", _clact_abs),
    "mean_wrong_divisor": ("token_mean", _mean_wrong_div),
    "bf16_truncation": ("round_to_dtype", _bf16_truncate),
    "relu2_squares_negatives": ("squared_relu", _relu2_abs),
    "relu2_not_rounded": ("squared_relu", _relu2_unrounded),
    "relu2_not_squared": ("squared_relu", _relu_only),
    "meta_lex_rank": ("comb_rank", _lex_rank),
    "amber_keeps_outliers": ("amber_factor", _amber_no_removal),
    "amber_raw_norm": ("amber_factor", _amber_raw_norm),
    "eta_table_last_value": ("eta_table", _eta_table_last),
    "ema_dense_denominator": ("var_factor_ema", _ema_dense_denominator),
    "e4m3_truncation": ("e4m3_round", _e4m3_truncate),
    "meta_width_floor": ("meta_width", _width_floor),
    "fp8_column_scales": ("fp8_rows", _fp8_column_scales),
    "fp8_inverted_scale": ("fp8_rows", _fp8_inverted_scale),
    "fp8_scale_over_whole_row": ("prefill_fp8", _fp8_whole_row_scale),
}


def _run_pin(fn):
    import inspect
    params = inspect.signature(fn).parameters
    marks = getattr(fn, "pytestmark", [])
    cases = [{}]
    for mk in marks:
        if mk.name == "parametrize":
            names = [s.strip() for s in mk.args[0].split(",")]
            vals = mk.args[1]
            cases = [dict(c, **dict(zip(names, v if len(names) > 1 else (v,)))) for c in cases for v in vals]
    for c in cases:
        fn(**{k: c[k] for k in params})


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_catches(mutant, monkeypatch):
    attr, fake = MUTANTS[mutant]
    monkeypatch.setattr(O, attr, fake)
    failures = []
    for name in PINS:
        try:
            _run_pin(getattr(P, name))
        except Exception:                                 # noqa: BLE001 - any failure counts
            failures.append(name)
            break
    assert failures, f"no pin failed with mutant {mutant}"

"""Pins of the CPU oracle to facts other than itself (CPU only).

Each test checks an oracle function against something the pages or plain
mathematics fix: values the pages print, closed forms, brute force over all
subsets, exact rational arithmetic, invariants, or an independent library
routine.  A plausible slip in the oracle (a dropped term, a flipped sign or
comparison, a transposed operand, a wrong tie order) fails at least one.
"""
import itertools
import json
import math
import os
import statistics
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nm_oracle as O
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


def _x32(t):
    return t.float().numpy()


# --------------------------------------------------------------------------
# top-N rule
# --------------------------------------------------------------------------

def _brute_force_keep(scores_block, n):
    """Best n-subset by exact sum; ties broken by the smallest sorted index tuple."""
    best = None
    for sub in itertools.combinations(range(len(scores_block)), n):
        tot = sum(Fraction(float(scores_block[i])) for i in sub)
        key = (tot, tuple(-i for i in sub))
        if best is None or key > best[0]:
            best = (key, sub)
    return set(best[1])


@pytest.mark.parametrize("n,m", [(1, 4), (2, 4), (3, 4), (4, 4), (2, 8), (4, 8), (5, 8), (8, 16), (3, 16)])
def test_topn_matches_brute_force(n, m):
    rng = np.random.Generator(np.random.PCG64(n * 100 + m))
    blocks = [
        rng.random(m).astype(np.float32),
        np.full(m, 0.5, np.float32),
        np.zeros(m, np.float32),
        rng.choice(np.array([0.0, 0.25, 1.0], np.float32), m),
        np.abs(np.repeat(rng.standard_normal(m // 2), 2)).astype(np.float32),
    ]
    one_big = np.full(m, 0.25, np.float32)
    one_big[m // 3] = 4.0
    blocks.append(one_big)
    sc = np.stack(blocks)
    keep = O.topn_mask(sc, n, m)
    for r in range(sc.shape[0]):
        got = set(np.nonzero(keep[r])[0].tolist())
        assert got == _brute_force_keep(sc[r], n), (r, sc[r])


def test_subset_counts_match_printed_table():
    tab = _gold("nm_pattern_table.json")["rows"]
    for row in tab:
        c = math.comb(row["m"], row["n"])
        if row["combinations"] is not None:
            assert c == row["combinations"]
            if row["m"] <= 16:
                assert sum(1 for _ in itertools.combinations(range(row["m"]), row["n"])) == c
        else:
            # printed as "6x10^8"
            assert c == 601080390 and round(c / 1e8) == 6


def test_metadata_bits_match_printed_table():
    # Information content of one block, ceil(log2 C(m,n)) bits, spread over m elements.
    tab = _gold("nm_pattern_table.json")["rows"]
    for row in tab:
        bits = math.ceil(math.log2(math.comb(row["m"], row["n"]))) / row["m"]
        if row["pattern"] == "4:8":
            # printed 0.81; ceil(log2 70)/8 = 0.875 and log2(70)/8 = 0.766: a slip on the page
            assert bits == 0.875
            continue
        assert round(bits, 2) == round(row["bits_per_element"], 2), row


def test_tie_rule_examples():
    for case in _gold("tie_rule_examples.json")["cases"]:
        sc = np.array([case["scores"]], np.float32)
        keep = O.topn_mask(sc, case["n"], case["m"])
        assert np.nonzero(keep[0])[0].tolist() == case["kept"]
        _, idx = O.pack(sc, keep, case["n"], case["m"], "f32")
        assert idx[0].tolist() == case["kept"]


@pytest.mark.parametrize("m", [4, 8, 16, 32])
def test_exactly_n_per_block(m):
    rng = np.random.Generator(np.random.PCG64(m))
    for n in sorted({1, m // 4 or 1, m // 2, m - 1, m}):
        for kind in ["random", "equal", "zeros", "signed_pairs", "signed_zero", "one_big", "few_levels"]:
            if kind == "random":
                x = rng.standard_normal((5, 4 * m)).astype(np.float32)
            else:
                x = _x32(wl.adversarial_x(kind, 5, 4 * m, m, "f32", seed=m))
            keep = O.topn_mask(O.scores(x, None), n, m)
            assert (keep.reshape(5, 4, m).sum(-1) == n).all(), (n, kind)


def test_tie_free_mask_equals_page_threshold_rule():
    # Magnitude code of the guide, s2.2.1: keep |x| >= the n-th largest |x| of its block.
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.standard_normal((64, 256)).astype(np.float32)
    for n, m in [(2, 4), (4, 8), (8, 16), (16, 32)]:
        blocks = np.abs(x).reshape(64, -1, m)
        assert all(len(set(b.tolist())) == m for b in blocks.reshape(-1, m))  # tie free
        thr = -np.sort(-blocks, axis=-1)[..., n - 1:n]
        page = (blocks >= thr).reshape(64, 256)
        assert (O.topn_mask(O.scores(x, None), n, m) == page).all()


# --------------------------------------------------------------------------
# shift, scores, rescale
# --------------------------------------------------------------------------

def test_token_mean_exact_rational():
    rng = np.random.Generator(np.random.PCG64(11))
    x = rng.standard_normal((3, 16)).astype(np.float32) * np.float32(3.0)
    eta = O.token_mean(x)
    for i in range(3):
        exact = sum(Fraction(float(v)) for v in x[i]) / 16
        assert eta[i] == np.float32(float(exact))  # one rounding of the exact mean (K a power of 2)


def test_token_mean_order_stable_on_workloads():
    # The mean is the exact sum rounded once; on the decode/prefill inputs a
    # float64 sum in any order gives the same value.
    for name in ["decode", "prefill"]:
        spec = wl.SPECS[name].with_(t=min(wl.SPECS[name].t, 16))
        x, _ = wl.make_inputs(spec, with_weight=False)
        x = _x32(x).astype(np.float64)
        eta = O.token_mean(x)
        for order in [slice(None), slice(None, None, -1)]:
            naive = np.array([np.float32(float(np.add.reduce(r[order], dtype=np.float64)) / x.shape[1]) for r in x])
            assert (naive == eta).all()
        pairwise = np.float32(x.sum(axis=1) / x.shape[1])
        assert (pairwise == eta).all()


def test_shift_identity_pages_form():
    # (x_hat*m + eta) W^T  ==  (x_hat*m) W^T + eta * (W 1)
    spec = wl.SPECS["prefill"].with_(t=6, k=64, n_out=24, n_outliers=2)
    x, w = wl.make_inputs(spec, seed=3)
    x, w = _x32(x), _x32(w)
    pr = O.prune(x, "bf16", 2, 4, shift_mode="token_mean")
    assert np.abs(pr["eta"]).max() > 0
    a = O.linear(pr, w)
    b = O.linear_pages_form(pr, w)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(b).max()
    # dropping the shift term must be visible
    pr0 = dict(pr, eta=np.zeros_like(pr["eta"]))
    assert np.abs(O.linear(pr0, w) - b).max() > 1e-3 * np.abs(b).max()


def test_n_equals_m_reproduces_dense_exact():
    rng = np.random.Generator(np.random.PCG64(2))
    x = rng.standard_normal((2, 8)).astype(np.float32)
    w = rng.standard_normal((3, 8)).astype(np.float32)
    pr = O.prune(x, "f32", 4, 4)
    assert pr["keep"].all()
    assert (pr["idx"].reshape(2, 2, 4) == np.arange(4)).all()
    y = O.linear(pr, w)
    for i in range(2):
        for j in range(3):
            exact = sum(Fraction(float(x[i, c])) * Fraction(float(w[j, c])) for c in range(8))
            assert abs(Fraction(float(y[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 60)


def test_n_equals_m_with_shift_matches_torch_dense():
    spec = wl.SPECS["decode"].with_(t=3, k=256, n_out=40)
    x, w = wl.make_inputs(spec, seed=1)
    pr = O.prune(_x32(x), "bf16", 16, 16, shift_mode="token_mean")
    y = O.linear(pr, _x32(w))
    dense = (x.double() @ w.double().T).numpy()
    assert O.rowwise_error(y, dense) <= 1e-6


def test_var_factor_closed_form_rational():
    rng = np.random.Generator(np.random.PCG64(4))
    x = rng.laplace(0, 0.3, size=(3, 32)).astype(np.float32)
    pr = O.prune(x, "f32", 4, 8, var_rescale=True)
    for i in range(3):
        full = [Fraction(float(v)) for v in pr["xhat"][i]]
        kept = [v if k else Fraction(0) for v, k in zip(full, pr["keep"][i])]
        ratio = statistics.pvariance(full) / statistics.pvariance(kept)
        assert abs(float(pr["nu"][i]) - math.sqrt(ratio)) <= 1e-6 * math.sqrt(ratio)
        assert pr["nu"][i] > 1.0      # pruning removes variance


def test_var_factor_degenerate():
    x = np.zeros((2, 8), np.float32)
    x[1, 3] = 1.0
    pr = O.prune(x, "f32", 2, 4, var_rescale=True)
    assert pr["nu"][0] == 1.0                      # all-zero row: 0/0 -> 1
    assert abs(pr["nu"][1] - 1.0) < 1e-7           # the single non-zero is kept: ratio 1


def test_nu_rescales_output():
    rng = np.random.Generator(np.random.PCG64(8))
    x = rng.laplace(0, 0.3, (2, 64)).astype(np.float32)
    w = rng.normal(0, 0.02, (5, 64)).astype(np.float32)
    pr = O.prune(x, "f16", 16, 32, score="clact", var_rescale=True)
    y = O.linear(pr, w)
    plain = (pr["xhat"].astype(np.float64) * pr["keep"]) @ w.astype(np.float64).T
    assert np.allclose(y, pr["nu"][:, None].astype(np.float64) * plain, rtol=1e-12, atol=0)


def test_weight_factor_independent_norm():
    spec = wl.SPECS["decode"].with_(k=96, n_out=300)
    _, w = wl.make_inputs(spec)
    w32 = _x32(w)
    for alpha in [0.0, 0.5, 1.0, 0.3]:
        f = O.channel_factor(w32, alpha)
        ref = torch.linalg.vector_norm(w.double(), dim=0) ** alpha
        assert np.allclose(f, ref.numpy(), rtol=2 ** -23, atol=0)
    assert (O.channel_factor(w32, 0.0) == 1.0).all()


def test_weight_factor_exact_tiny():
    w = np.array([[3.0, 1.0], [4.0, 1.0]], np.float32)
    assert O.channel_factor(w, 1.0).tolist() == [5.0, np.float32(math.sqrt(2.0))]
    assert O.channel_factor(w, 2.0).tolist() == [25.0, 2.0]
    assert O.row_sum(w).tolist() == [4.0, 5.0]


def test_weight_aware_uses_column_norm_of_w():
    # The factor multiplies input channel k by the norm of W's column k (outputs),
    # so a channel whose weights are large survives against a larger activation.
    x = np.array([[1.0, 0.9, 0.1, 0.1]], np.float32)
    w = np.ones((3, 4), np.float32)
    w[:, 1] = 4.0
    f = O.channel_factor(w, 1.0)
    pr_w = O.prune(x, "f32", 1, 4, score="weight", f=f)
    pr_m = O.prune(x, "f32", 1, 4)
    assert pr_m["idx"].tolist() == [[0]]
    assert pr_w["idx"].tolist() == [[1]]


def test_alpha_zero_equals_magnitude():
    spec = wl.SPECS["decode"].with_(t=4, k=512, n_out=64)
    x, w = wl.make_inputs(spec)
    f = O.channel_factor(_x32(w), 0.0)
    a = O.prune(_x32(x), "bf16", 8, 16, score="weight", f=f, shift_mode="token_mean")
    b = O.prune(_x32(x), "bf16", 8, 16, score="magnitude", shift_mode="token_mean")
    assert (a["keep"] == b["keep"]).all() and (a["vals"] == b["vals"]).all()


def test_clact_single_token_equals_magnitude():
    spec = wl.SPECS["batched"].with_(t=1, k=1024)
    x, _ = wl.make_inputs(spec, with_weight=False)
    x = _x32(x)
    c = O.clact_colnorm(x)
    assert (c == np.abs(x[0])).all()   # fp16 squares are exact in fp32; sqrt of a square
    a = O.prune(x, "f16", 16, 32, score="clact")
    b = O.prune(x, "f16", 16, 32)
    assert (a["keep"] == b["keep"]).all()


def test_clact_colnorm_vs_float64_norm():
    spec = wl.SPECS["batched"].with_(t=32, k=2048)
    x, _ = wl.make_inputs(spec, with_weight=False)
    x = _x32(x)
    c = O.clact_colnorm(x)
    ref = np.sqrt((x.astype(np.float64) ** 2).sum(axis=0))
    assert np.allclose(c, ref, rtol=32 * 2 ** -24, atol=0)


def test_clact_row_factor_does_not_change_masks():
    # The page's CLACT score also divides by the row norm ||x_i||.
    spec = wl.SPECS["batched"].with_(t=8, k=2048)
    x, _ = wl.make_inputs(spec, with_weight=False)
    x = _x32(x)
    pr = O.prune(x, "f16", 16, 32, score="clact")
    x64 = x.astype(np.float64)
    full = np.abs(x64) / np.sqrt((x64 ** 2).sum(axis=1, keepdims=True)) * np.sqrt((x64 ** 2).sum(axis=0))
    keep_full = O.topn_mask(full.astype(np.float32), 16, 32)
    assert (keep_full != pr["keep"]).sum() == 0


def test_scale_by_power_of_two_invariant():
    rng = np.random.Generator(np.random.PCG64(9))
    x = rng.standard_normal((4, 128)).astype(np.float32)
    for n, m in [(2, 4), (8, 16), (16, 32)]:
        a = O.topn_mask(O.scores(x, None), n, m)
        b = O.topn_mask(O.scores(x * np.float32(8.0), None), n, m)
        c = O.topn_mask(O.scores(x * np.float32(0.0625), None), n, m)
        assert (a == b).all() and (a == c).all()


def test_score_uses_shifted_value():
    # Under a shift the score is |x - eta|: a value equal to the mean is pruned first.
    x = np.array([[1.0, 1.0, 1.0, 5.0, 3.0, 3.0, 3.0, 3.0]], np.float32)
    pr = O.prune(x, "f32", 1, 4, shift_mode="token_mean")
    assert pr["eta"][0] == 2.5
    # block 1 scores 1.5,1.5,1.5,2.5 -> position 3; block 2 all 0.5 -> position 0
    assert pr["idx"].tolist() == [[3, 0]]
    assert np.array_equal(pr["vals"][0], np.array([2.5, 0.5], np.float32))


# --------------------------------------------------------------------------
# pack and storage rounding
# --------------------------------------------------------------------------

def test_pack_reconstructs_masked_values():
    spec = wl.SPECS["relu2"].with_(t=16, k=256)
    x, _ = wl.make_inputs(spec, with_weight=False)
    x = _x32(x)
    for dtype in ["bf16", "f16", "f32"]:
        pr = O.prune(x, dtype, 2, 4)
        dense = np.zeros_like(x)
        blk = np.repeat(np.arange(x.shape[1] // 4) * 4, 2)[None, :]
        np.put_along_axis(dense, blk + pr["idx"].astype(np.int64), pr["vals"], axis=1)
        assert np.array_equal(dense, O.round_to_dtype(x, dtype) * pr["keep"])
        assert (np.diff(pr["idx"].reshape(16, -1, 2).astype(int), axis=-1) > 0).all()


@pytest.mark.parametrize("dtype,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_round_to_dtype_matches_torch(dtype, tdt):
    rng = np.random.Generator(np.random.PCG64(1))
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-3).astype(np.float32),
        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 2 ** -8)], np.float32),
    ])
    # exact bf16 halfway points: low 16 bits == 0x8000
    halves = (rng.integers(0x3F000000, 0x40800000, 500, dtype=np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    v = np.concatenate([v, halves.view(np.float32)])
    ref = torch.from_numpy(v).to(tdt).float().numpy()
    got = O.round_to_dtype(v, dtype)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------------------
# FP8 (e4m3)
# --------------------------------------------------------------------------

def test_e4m3_codes_follow_the_format():
    # the 256 codes from the OCP e4m3 definition, spot values by hand
    assert O.e4m3_value(0x38) == 1.0 and O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0x01) == 2.0 ** -9
    assert O.e4m3_value(0x08) == 2.0 ** -6 and O.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert math.isnan(O.e4m3_value(0x7F)) and math.isnan(O.e4m3_value(0xFF))
    vals = [O.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))                 # codes ordered like values
    assert all(O.e4m3_value(c | 0x80) == -O.e4m3_value(c) for c in range(0x7F))


def test_e4m3_round_is_nearest_even_by_exhaustive_search():
    rng = np.random.Generator(np.random.PCG64(12))
    reps = [O.e4m3_value(c) for c in range(0x7F)]
    mids = [(a + b) / 2 for a, b in zip(reps, reps[1:])]
    x = np.concatenate([rng.uniform(-460, 460, 3000), rng.standard_normal(500) * 1e-2, reps, mids,
                        np.negative(mids), [0.0, -0.0, 448.0, 464.0 - 1e-3, -1e-5, -2.0 ** -11, 2.0 ** -11]]).astype(np.float32)
    got = O.e4m3_round(x)
    for xi, ci in zip(x.tolist(), got.tolist()):
        cand = [(abs(Fraction(O.e4m3_value(c)) - abs(Fraction(xi))), c & 1, c) for c in range(0x7F)]
        best = min(cand)[2]
        want = best | (0x80 if math.copysign(1.0, xi) < 0 else 0)     # signed zeros keep the sign
        assert ci == want, (xi, hex(ci), hex(want))


def test_fp8_rows_scale_and_extremes():
    v = np.array([[0.5, -2.0, 1.0, 0.0], [0, 0, 0, 0], [3.0, 3.0, -3.0, 1e-3]], dtype=np.float32)
    q, s = O.fp8_rows(v)
    assert s[1] == 0 and (q[1] == 0).all()
    assert O.e4m3_value(int(q[0, 1])) == -448.0 and O.e4m3_value(int(q[2, 0])) == 448.0
    assert s[0] == np.float32(2.0 / 448.0)
    # dequantised values within half an e4m3 step (relative 1/16) of the input
    deq = O.e4m3_decode(q) * s[:, None]
    big = np.abs(v) > 0.05
    assert np.all(np.abs(deq[big] - v[big]) <= np.abs(v[big]) / 16 + 1e-12)


def test_prefill_fp8_lossless_case_is_the_exact_product():
    # integers in [-7, 7] with a 7 in every row: the scales are 7 / 448 = 1 / 64
    # and every scaled value 64 v is an e4m3 value, so the FP8 product equals
    # the exact integer product of the kept entries
    rng = np.random.Generator(np.random.PCG64(31))
    x = rng.integers(-7, 8, size=(5, 64))
    w = rng.integers(-7, 8, size=(6, 64))
    x[:, 3], w[:, 10] = 7, -7
    pr = O.prefill_fp8(x.astype(np.float32), w.astype(np.float32), "bf16")
    assert (pr["sx"] == np.float32(1 / 64)).all() and (pr["sw"] == np.float32(1 / 64)).all()
    keep = pr["keep"].astype(np.int64)
    assert np.array_equal(keep.reshape(5, 16, 4).sum(-1), np.full((5, 16), 2))
    exact = (x * keep) @ w.T
    assert np.array_equal(pr["y"], exact.astype(np.float64))


def test_prefill_fp8_scale_is_over_the_kept_entries():
    # [SqReLU] s5.3: sparsify, then quantise.  With the weight-aware score a
    # row's largest |x_hat| can be pruned (a tiny channel factor); the token's
    # scale is then the largest KEPT |x_hat| / 448, and that entry codes to
    # +-448 exactly (0x7E / 0xFE)
    x = np.array([[10.0, 1.0, 2.0, 0.5, -3.0, 0.25, 1.5, 0.75],
                  [0.5, -9.0, 0.25, 1.0, 0.0, 0.0, 0.0, 0.0]], np.float32)
    f = np.array([1e-3, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0], np.float32)
    w = np.eye(8, dtype=np.float32)
    pr = O.prefill_fp8(x, w, "f32", score="weight", f=f)
    assert not pr["keep"][0, 0] and pr["keep"][0, 2] and pr["keep"][0, 4]
    assert pr["sx"][0] == np.float32(3.0) / np.float32(448.0)
    assert pr["qx"][0, 4] == 0xFE and pr["qx"][0, 2] != 0
    assert pr["sx"][1] == np.float32(9.0) / np.float32(448.0) and pr["qx"][1, 1] == 0xFE
    # on a workload sample: every row's largest kept code is +-448
    spec = wl.SPECS["prefill"].with_(t=12, k=256, n_out=8, score="weight", alpha=1.0, n_outliers=0)
    xs, ws = wl.make_inputs(spec)
    xs[:, 7] = 20.0                          # each row's largest value, on a channel of tiny weights
    ws[:, 7] *= 1e-3
    fa = O.channel_factor(_x32(ws), 1.0)
    pr = O.prefill_fp8(_x32(xs), _x32(ws), "bf16", score="weight", f=fa, shift_mode="token_mean")
    mags = np.abs(O.e4m3_decode(pr["qx"]))
    assert (mags.max(axis=1) == 448.0).all()
    xh = np.abs(pr["xhat"])
    assert (np.where(pr["keep"], xh, 0).max(axis=1) < xh.max(axis=1)).all()   # the readings differ here


def test_prefill_fp8_close_to_bf16():
    # FP8 quantisation error of y against the 16-bit product: a few per cent
    spec = wl.SPECS["prefill"].with_(t=16, k=512, n_out=64)
    x, w = wl.make_inputs(spec)
    pr8 = O.prefill_fp8(_x32(x), _x32(w), "bf16", shift_mode="token_mean")
    pr = O.prune(_x32(x), "bf16", 2, 4, shift_mode="token_mean")
    assert np.array_equal(pr8["keep"], pr["keep"])
    assert O.rowwise_error(pr8["y"], O.linear(pr, _x32(w))) < 0.08


# --------------------------------------------------------------------------
# squared-ReLU FFN
# --------------------------------------------------------------------------

def test_ffn_relu2_small_exact():
    # integer inputs: the up-projection is exact, so u, its square, the mask
    # and the output follow from integer arithmetic
    rng = np.random.Generator(np.random.PCG64(8))
    x = rng.integers(-3, 4, size=(3, 16)).astype(np.float32)
    w_up = rng.integers(-2, 3, size=(8, 16)).astype(np.float32)
    w_dn = rng.integers(-2, 3, size=(5, 8)).astype(np.float32)
    pr = O.ffn_relu2(x, w_up, w_dn, "bf16")
    u = x.astype(np.int64) @ w_up.astype(np.int64).T
    # the activation is stored in bf16: each square rounded once (exact rationals)
    a = np.array([[_round_exact(Fraction(int(v)) ** 2, "bf16") if v > 0 else 0.0 for v in row] for row in u])
    assert np.array_equal(pr["u"], u.astype(np.float32))
    for i in range(3):
        for b in range(2):
            blk = a[i, 4 * b:4 * b + 4]
            order = sorted(range(4), key=lambda j: (-blk[j], j))[:2]
            assert sorted(order) == list(pr["idx"][i, 2 * b:2 * b + 2])
    keep = np.zeros_like(a)
    for i in range(3):
        for b in range(2):
            for j in pr["idx"][i, 2 * b:2 * b + 2]:
                keep[i, 4 * b + j] = a[i, 4 * b + j]
    y = [[float(sum(Fraction(keep[i, c]) * int(w_dn[o, c]) for c in range(8))) for o in range(5)] for i in range(3)]
    assert np.array_equal(pr["y"], np.array(y))


# --------------------------------------------------------------------------
# running-average variance factor
# --------------------------------------------------------------------------

def test_var_ema_exact_small():
    # x_hat rows of small integers: the variances are exact rationals
    xh = np.array([[1, -2, 3, 0, 4, -1, 2, 5], [2, 2, -2, -2, 1, 0, 0, 3]], dtype=np.float32)
    keep = np.array([[1, 0, 1, 0, 1, 0, 0, 1], [1, 1, 1, 1, 0, 0, 0, 0]], dtype=bool)
    r_in = np.array([2.5, 0.75], dtype=np.float32)
    nu, r = O.var_factor_ema(xh, keep, r_in)
    for i in range(2):
        vals = [Fraction(int(v)) for v in xh[i]]
        kept = [v if k else Fraction(0) for v, k in zip(vals, keep[i])]
        var = lambda a: sum(v * v for v in a) / len(a) - (sum(a) / len(a)) ** 2
        r_want = Fraction(9, 10) * Fraction(float(r_in[i])) + Fraction(1, 10) * var(vals)
        nu_want = math.sqrt(float(r_want / (var(kept) + Fraction(1, 10 ** 6))))
        assert abs(float(r[i]) - float(r_want)) <= 1e-7 * float(r_want)
        assert abs(float(nu[i]) - nu_want) <= 1e-6 * nu_want


def test_var_ema_steady_state_matches_closed_form():
    # with the state at the dense variance, the state stays and nu is the
    # closed form times sqrt(D / (D + 1e-6))
    spec = wl.SPECS["batched"].with_(t=8, k=2048)
    x, _ = wl.make_inputs(spec, with_weight=False)
    pr = O.prune(_x32(x), "f16", 16, 32)
    v = pr["xhat"].astype(np.float64).var(axis=1)
    d = (pr["xhat"].astype(np.float64) * pr["keep"]).var(axis=1)
    nu, r = O.var_factor_ema(pr["xhat"], pr["keep"], v)
    assert np.allclose(r, v, rtol=1e-6, atol=0)
    closed = O.var_factor(pr["xhat"], pr["keep"]).astype(np.float64)
    assert np.allclose(nu, closed * np.sqrt(d / (d + 1e-6)), rtol=1e-6, atol=0)


# --------------------------------------------------------------------------
# S-PTS table
# --------------------------------------------------------------------------

def test_eta_table_exact_means():
    # rows of a constant value c have shift exactly c; an id's entry is the
    # exact average of its rows' constants, rounded once
    consts = [0.5, -1.25, 3.0, 0.75, 2.0, -0.5, 0.125]
    ids = [3, 0, 3, 5, 3, 0, 1]
    x = np.array([[c] * 64 for c in consts], dtype=np.float32)
    tab = O.eta_table([(x[:4], ids[:4]), (x[4:], ids[4:])], vocab=6)
    for v in range(6):
        vals = [Fraction(c) for c, i in zip(consts, ids) if i == v]
        want = np.float32(float(sum(vals) / len(vals))) if vals else np.float32(0.0)
        assert tab[v] == want, (v, tab[v], want)
    assert list(O.eta_lookup(tab, [3, 0, 9, -1, 5])) == [tab[3], tab[0], 0.0, 0.0, tab[5]]


def test_eta_table_single_occurrence_is_the_dynamic_shift():
    spec = wl.SPECS["prefill"].with_(t=16, k=512)
    x, _ = wl.make_inputs(spec, with_weight=False)
    x = _x32(x)
    tab = O.eta_table([(x, np.arange(16))], vocab=16)
    for i in range(16):
        exact = sum(Fraction(float(v)) for v in x[i]) / 512
        assert tab[i] == np.float32(float(exact))


# --------------------------------------------------------------------------
# Amber-Pruner channel factor
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed,n", [(0, 400), (1, 1001), (2, 65536), (3, 7)])
def test_amber_percentile_matches_numpy(seed, n):
    v = np.sort(np.random.Generator(np.random.PCG64(seed)).standard_normal(n))
    for q in (0.5, 99.5, 50.0, 0.0, 100.0):
        ref = float(np.percentile(v, q, method="linear"))
        assert abs(O.percentile_linear(v, q) - ref) <= 2 * np.spacing(abs(ref))


def test_amber_removes_planted_outliers_exact():
    # 200 x 2 weights: two planted low and two planted high outliers fall
    # outside the 0.5 / 99.5 percentiles (order-statistic positions 1.995 and
    # 397.005 of 400); the factor is then the exact rational z-score norm of
    # the other 396 values
    rng = np.random.Generator(np.random.PCG64(4))
    w = np.round(rng.uniform(-1, 1, size=(200, 2)) * 64) / 64
    out = [(3, 0, -100.0), (77, 1, -90.0), (150, 0, 95.0), (9, 1, 120.0)]
    for j, c, v in out:
        w[j, c] = v
    keep = np.ones_like(w, dtype=bool)
    for j, c, _ in out:
        keep[j, c] = False
    vals = [Fraction(float(x)) for x in w[keep]]
    mean = sum(vals) / len(vals)
    var = sum((x - mean) ** 2 for x in vals) / len(vals)
    for alpha in (1.0, 0.5):
        f = O.amber_factor(w.astype(np.float32), alpha)
        for c in range(2):
            ss = sum((Fraction(float(x)) - mean) ** 2 for x in w[keep[:, c], c]) / var
            want = np.float32(float(ss) ** (alpha / 2))
            assert abs(float(f[c]) - float(want)) <= 2e-7 * float(want), (c, f[c], want)


def test_amber_invariant_to_scale_and_shift():
    rng = np.random.Generator(np.random.PCG64(5))
    w = (rng.standard_normal((300, 48)) * 0.02).astype(np.float32)
    w[rng.integers(0, 300, 6), rng.integers(0, 48, 6)] = 0.5          # a few outliers
    f = O.amber_factor(w, 1.0)
    assert np.array_equal(O.amber_factor(w * np.float32(4.0), 1.0), f)  # exact: a power of two
    g = O.amber_factor(w + np.float32(0.25), 1.0)                       # the mean is removed
    assert np.allclose(g, f, rtol=1e-5, atol=0)
    assert np.array_equal(O.amber_factor(w, 0.0), np.ones(48, np.float32))
    # the outliers are gone: one huge weight does not make its channel stand out
    w2 = w.copy()
    w2[0, 7] = 1e3
    assert abs(float(O.amber_factor(w2, 1.0)[7]) / float(f[7]) - 1.0) < 0.05


# --------------------------------------------------------------------------
# compact block metadata
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,m", [(1, 4), (2, 4), (3, 4), (4, 4), (2, 8), (4, 8), (7, 8), (3, 16), (8, 16),
                                 (1, 32), (2, 32), (31, 32)])
def test_comb_rank_is_colex_position(n, m):
    # enumerate every n-subset, sort them colexicographically (compare the
    # largest position first), and check that the rank is the list position
    subsets = sorted(itertools.combinations(range(m), n), key=lambda s: tuple(reversed(s)))
    for pos, sub in enumerate(subsets):
        assert O.comb_rank(sub) == pos
        assert O.comb_unrank(pos, n, m) == list(sub)
    assert len(subsets) == math.comb(m, n)


def test_comb_rank_order_16_of_32():
    # too many subsets to enumerate: the rank must order pairs as colex does
    rng = np.random.Generator(np.random.PCG64(11))
    top = math.comb(32, 16)
    for _ in range(400):
        a = tuple(sorted(rng.choice(32, 16, replace=False).tolist()))
        b = tuple(sorted(rng.choice(32, 16, replace=False).tolist()))
        ra, rb = O.comb_rank(a), O.comb_rank(b)
        assert 0 <= ra < top and 0 <= rb < top
        assert (ra < rb) == (tuple(reversed(a)) < tuple(reversed(b)))
        assert O.comb_unrank(ra, 16, 32) == list(a)


def test_meta_widths_match_printed_table():
    # bits per element printed in the pattern table (4:8's 0.81 is the page's
    # slip: 7 bits over 8 elements is 0.875) and 3 bits per 2:4 block
    table = {(2, 4): "0.75", (8, 16): "0.875", (16, 32): "0.94"}
    for (n, m), printed in table.items():
        digits = len(printed.split(".")[1])
        assert round(O.meta_width(n, m, "comb") / m, digits) == float(printed)
    assert O.meta_width(2, 4, "comb") == 3
    assert O.meta_width(4, 8, "comb") == 7
    assert O.meta_width(4, 4, "comb") == 0
    assert all(O.meta_width(n, m, "bitmap") == m for n, m in [(2, 4), (16, 32)])


def test_meta_golden_words():
    gold = _gold("meta_codes.json")
    for case in gold["cases"]:
        n, m, fmt = case["n"], case["m"], case["fmt"]
        idx = np.array(case["idx"], dtype=np.uint8)
        k = idx.shape[1] // n * m
        words = O.encode_meta(idx, n, m, fmt)
        assert words.tolist() == case["words"], case["derivation"]
        assert np.array_equal(O.decode_meta(words, k, n, m, fmt), idx)


@pytest.mark.parametrize("fmt", ["comb", "bitmap"])
@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (4, 8), (8, 16), (16, 32), (5, 32)])
def test_meta_round_trip_on_masks(fmt, n, m):
    spec = wl.SPECS["prefill"].with_(t=3, k=32 * 37)
    x, _ = wl.make_inputs(spec, with_weight=False)
    pr = O.prune(_x32(x), "bf16", n, m)
    words = O.encode_meta(pr["idx"], n, m, fmt)
    assert words.shape == (3, O.meta_row_words(spec.k, n, m, fmt))
    assert np.array_equal(O.decode_meta(words, spec.k, n, m, fmt), pr["idx"])
    if fmt == "bitmap":
        # the mask bits are the kept channels, block after block
        bits = np.unpackbits(words.view(np.uint8), axis=1, bitorder="little")[:, :spec.k].astype(bool)
        assert np.array_equal(bits, pr["keep"])


# --------------------------------------------------------------------------
# squared ReLU as the input transform
# --------------------------------------------------------------------------

# (significand bits, smallest normal exponent) of each storage format
_FORMATS = {"bf16": (8, -126), "f16": (11, -14), "f32": (24, -126)}
_MAXFIN = {"bf16": (2 - 2 ** -7) * 2.0 ** 127, "f16": 65504.0, "f32": float(np.finfo(np.float32).max)}


def _round_exact(v: Fraction, fmt: str) -> float:
    """Nearest value of ``fmt`` to the exact rational v >= 0, ties to the even significand."""
    if v == 0:
        return 0.0
    p, emin = _FORMATS[fmt]
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    e = max(e, emin)                                      # subnormals share the smallest ulp
    ulp = Fraction(2) ** (e - p + 1)
    q = v / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * ulp
    return math.inf if r > Fraction(_MAXFIN[fmt]) else float(r)


def _all_finite_16bit(dtype):
    bits = np.arange(1 << 16, dtype=np.uint32)
    if dtype == "bf16":
        v = (bits << np.uint32(16)).view(np.float32)
    else:
        v = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_squared_relu_every_16bit_value(dtype):
    # max(0, u)^2 for every finite value of the format, against the exact square
    # rounded once to the format by rational arithmetic
    u = _all_finite_16bit(dtype)
    with np.errstate(over="ignore"):
        got = O.squared_relu(u, dtype)
    want = np.array([_round_exact(Fraction(float(a)) ** 2 if a > 0 else Fraction(0), dtype) for a in u],
                    dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_squared_relu_float32_rounds_once():
    rng = np.random.Generator(np.random.PCG64(5))
    u = np.concatenate([rng.standard_normal(3000), rng.standard_normal(500) * 1e-20,
                        rng.standard_normal(500) * 1e15]).astype(np.float32)
    got = O.squared_relu(u, "f32")
    want = np.array([_round_exact(Fraction(float(a)) ** 2 if a > 0 else Fraction(0), "f32") for a in u],
                    dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert (got[u <= 0] == 0).all() and not np.signbit(got).any()


def test_squared_relu_feeds_the_pruning():
    # act="relu2" on u gives the same masks and values as pruning max(0, u)^2
    # written out with exact rational squares
    spec = wl.SPECS["relu2_fused"].with_(t=4, k=256)
    u, _ = wl.make_inputs(spec, with_weight=False)
    u = _x32(u)
    x = np.array([[_round_exact(Fraction(float(a)) ** 2 if a > 0 else Fraction(0), "bf16") for a in row]
                  for row in u], dtype=np.float32)
    a = O.prune(u, "bf16", 2, 4, shift_mode="token_mean", act="relu2")
    b = O.prune(x, "bf16", 2, 4, shift_mode="token_mean")
    assert np.array_equal(a["keep"], b["keep"]) and np.array_equal(a["vals"], b["vals"])
    assert np.array_equal(a["eta"], b["eta"])


def test_squared_relu_of_preactivation_closed_form():
    # z ~ N(-1, 1): max(0, z)^2 is zero with probability Phi(1) = 0.8413
    spec = wl.SPECS["relu2_fused"].with_(t=256, k=4096)
    u, _ = wl.make_inputs(spec, with_weight=False)
    x = O.squared_relu(_x32(u), "bf16")
    p = 0.5 * math.erfc(1.0 / math.sqrt(2.0))
    assert abs(float((x == 0).mean()) - (1 - p)) < 0.002
    gold = _gold("squared_relu_sparsity.json")
    spec = wl.SPECS["prefill"].with_(t=256, k=4096, n_outliers=0)
    z, _ = wl.make_inputs(spec, with_weight=False)
    frac = float((O.squared_relu(_x32(z), "bf16") == 0).mean())
    assert abs(frac - gold["zero_fraction_standard_normal"]) < 0.005


# --------------------------------------------------------------------------
# workload statistics (generator and mask together)
# --------------------------------------------------------------------------

def test_squared_relu_standard_normal_half_zeros():
    gold = _gold("squared_relu_sparsity.json")
    spec = wl.SPECS["relu2"].with_(t=256, k=4096, x_dist="relu2_standard")
    x, _ = wl.make_inputs(spec, with_weight=False)
    frac = float((x == 0).float().mean())
    assert abs(frac - gold["zero_fraction_standard_normal"]) < 0.005


def test_relu2_workload_statistics_closed_form():
    spec = wl.SPECS["relu2"].with_(t=512)
    x, _ = wl.make_inputs(spec, with_weight=False)
    x = _x32(x)
    p = 0.5 * math.erfc(1.0 / math.sqrt(2.0))           # P(z > 0), z ~ N(-1, 1)
    zeros = float((x == 0).mean())
    assert abs(zeros - (1 - p)) < 0.002
    pr = O.prune(x, "bf16", 2, 4)
    nz = (x != 0)
    dropped = float((nz & ~pr["keep"]).sum()) / float(nz.sum())
    p3 = 4 * p ** 3 * (1 - p)
    p4 = p ** 4
    expect = (p3 * 1 + p4 * 2) / (4 * p)
    assert abs(dropped - expect) < 0.002                # about 2.3 % of non-zeros
    # the mask never prefers a zero over a non-zero
    blocks_nz = nz.reshape(512, -1, 4).sum(-1)
    kept_nz = (nz & pr["keep"]).reshape(512, -1, 4).sum(-1)
    assert (kept_nz == np.minimum(blocks_nz, 2)).all()


def test_workload_shapes_and_outliers():
    spec = wl.SPECS["decode"]
    x, _ = wl.make_inputs(spec, with_weight=False)
    assert x.shape == (1, 4096) and x.dtype == torch.bfloat16
    # recipe: base values, then the outlier columns, each multiplied by the gain
    rng = np.random.Generator(np.random.PCG64(0))
    base = 0.5 * rng.standard_t(3.0, size=(1, 4096))
    cols = rng.choice(4096, 8, replace=False)
    base[:, cols] *= 20.0
    ref = torch.from_numpy(base.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(x, ref)
    assert float(x[0, cols].float().abs().mean()) > 10 * float(x.float().abs().mean())
    spec = wl.SPECS["prefill"].with_(t=64)
    x, _ = wl.make_inputs(spec, with_weight=False)
    col_rms = x.float().pow(2).mean(0).sqrt()
    assert int((col_rms > 5).sum()) == 41

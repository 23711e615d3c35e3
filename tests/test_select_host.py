"""The library's per-block selection network, compiled for the host, against the oracle's rank rule (CPU only)."""
import itertools
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import nm_oracle as O
import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("sel") / "select_driver")
    subprocess.run([cxx, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "activation_sparsification_amd", "csrc"),
                    os.path.join(HERE, "native", "select_driver.cpp"), "-o", exe], check=True)
    return exe


def _run(exe, scores, n, m):
    blocks = scores.reshape(-1, m)
    inp = f"{m} {n} {blocks.shape[0]}\n" + " ".join(repr(float(v)) for v in blocks.ravel())
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split()
    bits = np.array([int(v) for v in out], dtype=np.uint64)
    return ((bits[:, None] >> np.arange(m, dtype=np.uint64)[None, :]) & 1).astype(bool)


@pytest.mark.parametrize("m", [4, 8, 16, 32])
def test_network_matches_rank_rule(driver, m):
    rng = np.random.Generator(np.random.PCG64(m))
    cases = [np.abs(rng.standard_normal((40, m))).astype(np.float32)]
    for kind in ["equal", "zeros", "signed_pairs", "signed_zero", "one_big", "few_levels"]:
        cases.append(np.abs(wl.adversarial_x(kind, 8, 4 * m, m, "f32", seed=m).float().numpy()).reshape(-1, m))
    cases.append(np.abs(rng.choice(np.array([0.0, 1.0, 2.0], np.float32), size=(40, m))))
    cases.append(np.full((2, m), 1e-42, np.float32))        # denormal ties
    sc = np.concatenate(cases).astype(np.float32)
    for n in sorted({1, 2, m // 2, m - 1, m}):
        if n < 1 or n > m:
            continue
        got = _run(driver, sc, n, m)
        want = O.topn_mask(sc, n, m)
        assert np.array_equal(got, want), (m, n)


def test_two_of_four_tournament_matches_rank_rule(driver):
    """The 2:4 tournament (four comparisons) keeps the same two positions as
    the rank rule, returns them in channel order with their values, and its
    code holds lo | hi << 2 with lo < hi: every block over the levels
    {0, 1, 2, 3} (all 256, which covers every pattern of ties), plus random
    and adversarial blocks."""
    levels = np.array(list(itertools.product(range(4), repeat=4)), dtype=np.float32)
    rng = np.random.Generator(np.random.PCG64(24))
    cases = [levels, np.abs(rng.standard_normal((200, 4))).astype(np.float32)]
    for kind in ["equal", "zeros", "signed_pairs", "signed_zero", "one_big", "few_levels"]:
        cases.append(np.abs(wl.adversarial_x(kind, 8, 16, 4, "f32", seed=4).float().numpy()).reshape(-1, 4))
    cases.append(np.full((2, 4), 1e-42, np.float32))
    sc = np.concatenate(cases).astype(np.float32)
    inp = f"0 2 {sc.shape[0]}\n" + " ".join(repr(float(v)) for v in sc.ravel())
    out = subprocess.run([driver], input=inp, capture_output=True, text=True, check=True).stdout.split()
    rows = np.array([int(v) for v in out], dtype=np.int64).reshape(-1, 4)
    keep = ((rows[:, 0:1] >> np.arange(4)[None, :]) & 1).astype(bool)
    want = O.topn_mask(sc, 2, 4)
    assert np.array_equal(keep, want)
    lo, hi, code = rows[:, 1], rows[:, 2], rows[:, 3]
    assert np.all(lo < hi)
    assert np.array_equal(code, lo | (hi << 2))
    assert np.array_equal(want[np.arange(len(lo)), lo] & want[np.arange(len(hi)), hi], np.ones(len(lo), bool))

"""GPU parity of the FP8 2:4 prefill against the oracle.

prepare_weight_fp8: codes and row scales bit for bit.  The pruned prefill
with FP8 operands: in-block positions bit for bit; the activation operand
the GEMM reads (per-token scales, every kept e4m3 code, the position words)
bit for bit, read back from the workspace; nu within 1e-6; y within the
16-bit tolerance of the oracle's FP8 product (the same e4m3 codes and
scales, summed in float64).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import nm_oracle as O
from gpu_util import f32, tiled_operand

pytestmark = pytest.mark.gpu

spa = pytest.importorskip("activation_sparsification_amd")


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a device"
    return torch.device("cuda:0")


def _cfg(spec):
    return spa.PruneConfig(spec.n, spec.m, spec.score, spec.shift, spec.var_rescale, spec.act)


@pytest.mark.parametrize("dtype,n_out,k", [("bf16", 300, 320), ("f16", 37, 64), ("bf16", 8, 1032)])
def test_prepare_weight_fp8(dtype, n_out, k):
    dev = _dev()
    spec = wl.SPECS["prefill"].with_(t=4, k=k, n_out=n_out, dtype=dtype, n_outliers=0)
    _, w = wl.make_inputs(spec)
    w[3] = 0                                                     # an all-zero row: scale 0, codes 0
    w[5, 7] = 30.0                                               # one large entry sets its row's scale
    w[5, 9] = -1e-6                                              # rounds to zero: the sign stays (0x80)
    w[6, 2] = -0.0
    print(f"[fp8 weight] {dtype} n_out={n_out} k={k}", flush=True)
    w8 = spa.prepare_weight_fp8(w.to(dev))
    torch.cuda.synchronize()
    q, s = O.fp8_rows(f32(w))
    assert np.array_equal(w8.codes.cpu().numpy(), q), "e4m3 codes differ"
    assert np.array_equal(f32(w8.scale).view(np.uint32), s.view(np.uint32)), "row scales differ"


FP8_CASES = [
    wl.SPECS["prefill"].with_(name="fp8_small", t=200, k=512, n_out=520, n_outliers=5),
    wl.SPECS["prefill"].with_(name="fp8_f16", t=77, k=320, n_out=300, dtype="f16", n_outliers=3),
    wl.SPECS["prefill"].with_(name="fp8_k64", t=5, k=64, n_out=40),
    wl.SPECS["prefill"].with_(name="fp8_k192", t=260, k=192, n_out=300),
    wl.SPECS["prefill"].with_(name="fp8_tiles", t=600, k=768, n_out=1100, n_outliers=8),
    wl.SPECS["prefill"].with_(name="fp8_one_row", t=1, k=128, n_out=8),
    # a last round of 192-column tiles (more 256 x 256 tiles than 256 CUs hold)
    wl.SPECS["prefill"].with_(name="fp8_tail_split", t=300, k=128, n_out=35000, n_outliers=2),
    wl.SPECS["prefill"].with_(name="fp8_weight_var", t=300, k=512, n_out=272, score="weight", alpha=0.5,
                              var_rescale=True),
    wl.SPECS["prefill"].with_(name="fp8_given", t=40, k=256, n_out=520, shift="given"),
    wl.SPECS["prefill"].with_(name="fp8_none", t=64, k=256, n_out=264, shift="none"),
    wl.SPECS["batched"].with_(name="fp8_clact", t=96, k=512, n_out=264, n=2, m=4),
    wl.SPECS["relu2_fused"].with_(name="fp8_relu2", t=136, k=1024, n_out=264),
    # every row's largest |x - eta| sits on a channel of tiny weights, which
    # the weight-aware score prunes: the token scale must come from the kept
    # entries (quantisation follows sparsification)
    wl.SPECS["prefill"].with_(name="fp8_weight_pruned_max", t=70, k=512, n_out=136, score="weight", alpha=1.0,
                              n_outliers=0),
]


def _fp8_oracle(spec, x, w, f=None, eta_in=None):
    if spec.score == "weight" and f is None:
        f = O.channel_factor(f32(w), spec.alpha)
    return O.prefill_fp8(f32(x), f32(w), spec.dtype, score=spec.score, f=f, shift_mode=spec.shift,
                         eta_in=None if eta_in is None else f32(eta_in), var_rescale=spec.var_rescale, act=spec.act)


def _fp8_inputs(spec):
    x, w = wl.make_inputs(spec)
    if spec.shift == "token_mean" and spec.t > 2:
        x[1] = x[1, 0]                                           # a constant row: x - eta == 0, scale 0
    if spec.name == "fp8_weight_pruned_max":
        x[:, 9] = 12.0
        w[:, 9] *= 1e-3
    return x, w


@pytest.mark.parametrize("spec", FP8_CASES, ids=[s.name for s in FP8_CASES])
def test_prefill_fp8_parity(spec):
    dev = _dev()
    x, w = _fp8_inputs(spec)
    eta_in = wl.make_eta(spec.t, 9) if spec.shift == "given" else None
    print(f"[fp8 prefill] {spec.name}: t={spec.t} k={spec.k} n_out={spec.n_out} {spec.score} {spec.shift}",
          flush=True)
    wd = w.to(dev)
    pw = spa.prepare_weight(wd, spec.alpha, want_wt=False)
    w8 = spa.prepare_weight_fp8(wd)
    f = f32(pw.chan_scale) if spec.score == "weight" else None
    if f is not None:
        assert np.array_equal(f.view(np.uint32), O.channel_factor(f32(w), spec.alpha).view(np.uint32))
    pr = _fp8_oracle(spec, x, w, f=f, eta_in=eta_in)
    cfg = _cfg(spec)
    ws = spa.workspace(2, spec.t, spec.k, spec.n_out, x.dtype, cfg, dev)
    y, idx, nu = spa.sparse_linear_prefill_fp8(x.to(dev), pw, w8, cfg,
                                               eta_in=None if eta_in is None else eta_in.to(dev), want_idx=True,
                                               want_nu=True, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), pr["idx"]), "FP8 prefill masks differ"
    assert np.allclose(f32(nu), pr["nu"], rtol=1e-6, atol=0)
    # the activation operand the GEMM read: per-token scales, every kept e4m3
    # code and the position words, bit for bit
    codes, pos, sx = tiled_operand(ws, spa.prefill_layout(spec.t, spec.k, x.dtype, cfg), spec.t, spec.k, True,
                                   spec.dtype)
    assert np.array_equal(sx.view(np.uint32), pr["sx"].view(np.uint32)), "FP8 token scales differ"
    keep = pr["keep"].reshape(spec.t, spec.k)
    want_codes = pr["qx"][keep].reshape(spec.t, spec.k // 2)
    assert np.array_equal(codes, want_codes), f"{int((codes != want_codes).sum())} e4m3 activation codes differ"
    assert np.array_equal(pos, pr["idx"]), "position words differ"
    if spec.name == "fp8_weight_pruned_max":                     # the two scale readings differ on every row
        amax = np.abs(pr["xhat"]).max(axis=1)
        nz = amax > 0
        assert (pr["sx"][nz] < amax[nz] / np.float32(448.0)).all()
    err = O.rowwise_error(f32(y), pr["y"])
    assert err <= O.TOLERANCE[spec.dtype], err


# Neither positions nor nu asked for, no variance factor (the benchmark's
# call): the lean pruning pass, here also on rows of two and four passes.
FP8_LEAN_CASES = [s for s in FP8_CASES if not s.var_rescale] + [
    wl.SPECS["prefill"].with_(name="fp8_k8192", t=21, k=8192, n_out=40),
    wl.SPECS["relu2_fused"].with_(name="fp8_k16384_mean", t=18, k=16384, n_out=40, shift="token_mean"),
]


@pytest.mark.parametrize("spec", FP8_LEAN_CASES, ids=[s.name for s in FP8_LEAN_CASES])
def test_prefill_fp8_operand_only(spec):
    dev = _dev()
    x, w = _fp8_inputs(spec)
    eta_in = wl.make_eta(spec.t, 9) if spec.shift == "given" else None
    print(f"[fp8 operand only] {spec.name}: t={spec.t} k={spec.k} n_out={spec.n_out}", flush=True)
    wd = w.to(dev)
    pw = spa.prepare_weight(wd, spec.alpha, want_wt=False)
    w8 = spa.prepare_weight_fp8(wd)
    f = f32(pw.chan_scale) if spec.score == "weight" else None
    pr = _fp8_oracle(spec, x, w, f=f, eta_in=eta_in)
    cfg = _cfg(spec)
    ws = spa.workspace(2, spec.t, spec.k, spec.n_out, x.dtype, cfg, dev)
    y, idx, nu = spa.sparse_linear_prefill_fp8(x.to(dev), pw, w8, cfg,
                                               eta_in=None if eta_in is None else eta_in.to(dev), ws=ws)
    torch.cuda.synchronize()
    assert idx is None and nu is None
    codes, pos, sx = tiled_operand(ws, spa.prefill_layout(spec.t, spec.k, x.dtype, cfg), spec.t, spec.k, True,
                                   spec.dtype)
    assert np.array_equal(pos, pr["idx"]), "position words differ"
    assert np.array_equal(sx.view(np.uint32), pr["sx"].view(np.uint32)), "FP8 token scales differ"
    want_codes = pr["qx"][pr["keep"].reshape(spec.t, spec.k)].reshape(spec.t, spec.k // 2)
    assert np.array_equal(codes, want_codes), f"{int((codes != want_codes).sum())} e4m3 activation codes differ"
    err = O.rowwise_error(f32(y), pr["y"])
    assert err <= O.TOLERANCE[spec.dtype], err


def test_prefill_fp8_rejections():
    dev = _dev()
    spec = wl.SPECS["prefill"].with_(t=8, k=256, n_out=64)
    x, w = wl.make_inputs(spec)
    wd = w.to(dev)
    pw = spa.prepare_weight(wd, 0.0, want_wt=False)
    w8 = spa.prepare_weight_fp8(wd)
    with pytest.raises(spa.SpaError) as e:                       # only 2:4 runs on the FP8 path
        spa.sparse_linear_prefill_fp8(x.to(dev), pw, w8, spa.PruneConfig(4, 8, shift="token_mean"))
    assert e.value.status == 2


@pytest.mark.parametrize("outputs", ["all", "operand"])
def test_prefill_fp8_full_size_sampled(outputs):
    # the prompt workload (2048 tokens, 4096 -> 14336) on sampled rows and
    # columns, with positions and nu asked for, and without (the lean pass)
    dev = _dev()
    spec = wl.SPECS["prefill"]
    print(f"[fp8 full size] t={spec.t} k={spec.k} n_out={spec.n_out}", flush=True)
    x, w = wl.make_inputs(spec)
    wd = w.to(dev)
    pw = spa.prepare_weight(wd, spec.alpha, want_wt=False)
    w8 = spa.prepare_weight_fp8(wd)
    cfg = _cfg(spec)
    wsp = spa.workspace(2, spec.t, spec.k, spec.n_out, x.dtype, cfg, dev)
    every = outputs == "all"
    y, idx, nu = spa.sparse_linear_prefill_fp8(x.to(dev), pw, w8, cfg, want_idx=every, want_nu=every, ws=wsp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.choice(spec.t, 24, replace=False), [0, spec.t - 1]]))
    cols = np.unique(np.concatenate([rng.choice(spec.n_out, 96, replace=False), [0, spec.n_out - 1]]))
    xs, ws = x[torch.as_tensor(rows)], w[torch.as_tensor(cols)]
    pr = _fp8_oracle(spec, xs, ws)
    if every:
        assert np.array_equal(idx.cpu().numpy()[rows], pr["idx"])
        assert np.allclose(f32(nu)[rows], pr["nu"], rtol=1e-6, atol=0)
    codes, pos, sx = tiled_operand(wsp, spa.prefill_layout(spec.t, spec.k, x.dtype, cfg), spec.t, spec.k, True,
                                   spec.dtype)
    assert np.array_equal(sx[rows].view(np.uint32), pr["sx"].view(np.uint32)), "FP8 token scales differ"
    want = pr["qx"][pr["keep"]].reshape(rows.size, spec.k // 2)
    assert np.array_equal(codes[rows], want), "e4m3 activation codes differ"
    assert np.array_equal(pos[rows], pr["idx"]), "position words differ"
    q, s = O.fp8_rows(f32(ws))
    assert np.array_equal(w8.codes.cpu().numpy()[cols], q)
    assert np.array_equal(f32(w8.scale)[cols].view(np.uint32), s.view(np.uint32))
    err = O.rowwise_error(f32(y)[np.ix_(rows, cols)], pr["y"])
    assert err <= O.TOLERANCE[spec.dtype], err


def test_prefill_fp8_max_k():
    # k = 2^23, the largest prefill k: a 256-row tile of weight codes spans
    # just under 2^31 bytes of 32-bit offsets
    dev = _dev()
    spec = wl.SPECS["prefill"].with_(t=3, k=1 << 23, n_out=256, n_outliers=0)
    print(f"[fp8 max size] t={spec.t} k={spec.k} n_out={spec.n_out}", flush=True)
    x, _ = wl.make_inputs(spec, with_weight=False)
    # the 2^31-element weight is drawn on the device (seeded); the oracle gets
    # copies of the sampled rows of that input
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    wd = torch.randn((spec.n_out, spec.k), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    torch.cuda.synchronize()
    pw = spa.prepare_weight(wd, 0.0, want_wt=False)
    w8 = spa.prepare_weight_fp8(wd)
    y, idx, _ = spa.sparse_linear_prefill_fp8(x.to(dev), pw, w8, _cfg(spec), want_idx=True)
    torch.cuda.synchronize()
    cols = np.array([0, 77, 200, spec.n_out - 1])               # the last row carries the largest offset
    ws = wd[torch.as_tensor(cols, device=dev)].cpu()
    pr = _fp8_oracle(spec, x, ws)
    assert np.array_equal(idx.cpu().numpy(), pr["idx"])
    q, s = O.fp8_rows(f32(ws))
    got = w8.codes[torch.as_tensor(cols, device=dev)].cpu().numpy()
    bad = np.argwhere(got != q)
    wv = f32(ws)
    detail = [(int(r), int(c), float(wv[r, c]), int(got[r, c]), int(q[r, c])) for r, c in bad[:8]]
    assert bad.shape[0] == 0, (bad.shape[0], detail, f32(w8.scale)[cols].tolist(), s.tolist())
    assert np.array_equal(f32(w8.scale)[cols].view(np.uint32), s.view(np.uint32))
    err = O.rowwise_error(f32(y)[:, cols], pr["y"])
    assert err <= O.TOLERANCE[spec.dtype], err


def test_prefill_fp8_running_average():
    # the running-average variance factor with caller-held state (in, out)
    dev = _dev()
    spec = wl.SPECS["prefill"].with_(t=300, k=512, n_out=272, n_outliers=0, var_rescale=2)
    x, w = wl.make_inputs(spec)
    r_in = np.random.Generator(np.random.PCG64(17)).uniform(0.05, 2.0, size=spec.t).astype(np.float32)
    st_in = torch.from_numpy(r_in).to(dev)
    st_out = torch.full((spec.t,), -1.0, dtype=torch.float32, device=dev)
    cfg = spa.PruneConfig(2, 4, spec.score, spec.shift, 2, spec.act, st_in, st_out)
    wd = w.to(dev)
    pw = spa.prepare_weight(wd, spec.alpha, want_wt=False)
    w8 = spa.prepare_weight_fp8(wd)
    y, idx, nu = spa.sparse_linear_prefill_fp8(x.to(dev), pw, w8, cfg, want_idx=True, want_nu=True)
    torch.cuda.synchronize()
    pr = O.prefill_fp8(f32(x), f32(w), spec.dtype, shift_mode=spec.shift, var_rescale=2, var_state=r_in)
    assert np.array_equal(idx.cpu().numpy(), pr["idx"])
    assert np.allclose(f32(nu), pr["nu"], rtol=1e-6, atol=0)
    assert np.allclose(f32(st_out), pr["var_state"], rtol=1e-6, atol=0)
    assert np.array_equal(f32(st_in), r_in)
    err = O.rowwise_error(f32(y), pr["y"])
    assert err <= O.TOLERANCE[spec.dtype], err


def test_prefill_fp8_workspace_reused():
    # one workspace, sized for the larger call, serves a larger then a smaller call
    dev = _dev()
    big = wl.SPECS["prefill"].with_(t=600, k=768, n_out=520, n_outliers=4)
    small = big.with_(t=45)
    x, w = wl.make_inputs(big)
    wd = w.to(dev)
    pw = spa.prepare_weight(wd, big.alpha, want_wt=False)
    w8 = spa.prepare_weight_fp8(wd)
    ws = spa.workspace(2, big.t, big.k, big.n_out, x.dtype, _cfg(big), dev)
    for spec, xs in ((big, x), (small, x[7:7 + small.t].contiguous())):
        y, idx, _ = spa.sparse_linear_prefill_fp8(xs.to(dev), pw, w8, _cfg(spec), want_idx=True, ws=ws)
        torch.cuda.synchronize()
        pr = _fp8_oracle(spec, xs, w)
        assert np.array_equal(idx.cpu().numpy(), pr["idx"]), spec.t
        err = O.rowwise_error(f32(y), pr["y"])
        assert err <= O.TOLERANCE[spec.dtype], (spec.t, err)

"""GPU parity at the benchmark's full sizes, through the calls the benchmark times.

- The weight factor prepare_weight returns must equal the oracle's bit for
  bit; the oracle then uses its own vector.
- Decode workloads (at most 32 tokens): positions bit for bit on every
  token, nu (1e-6 relative) on every token, y on every token and every
  output column against the float64 oracle (row-normwise, 2e-2 for 16-bit
  outputs).
- Prefill workloads, whose full product the oracle cannot form in seconds:
  positions checked on every row against what holds at any size (exactly n
  per block, ascending, inside the block) and bit for bit on sampled rows;
  nu on those rows; y on sampled rows x sampled columns.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import nm_oracle as O
from gpu_util import f32, storage_bits, tiled_operand

pytestmark = pytest.mark.gpu

spa = pytest.importorskip("activation_sparsification_amd")

FULL = {
    "decode": wl.SPECS["decode"],
    "prefill": wl.SPECS["prefill"],
    "relu2": wl.SPECS["relu2"],
    "relu2_fused": wl.SPECS["relu2_fused"],
    "batched_t1": wl.SPECS["batched"].with_(t=1),
    "batched_t8": wl.SPECS["batched"].with_(t=8),
    "batched_t32": wl.SPECS["batched"].with_(t=32),
}
DECODE = {"decode", "batched_t1", "batched_t8", "batched_t32"}


def _sample(total, count, seed):
    rng = np.random.default_rng(seed)
    pick = rng.choice(total, size=min(total, count), replace=False)
    return np.unique(np.concatenate([pick, [0, total - 1]]))


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled(name):
    assert torch.cuda.is_available(), "GPU tests need a device"
    dev = torch.device("cuda:0")
    spec = FULL[name]
    print(f"[full-size parity] {name}: t={spec.t} k={spec.k} n_out={spec.n_out} {spec.n}:{spec.m}", flush=True)
    x, w = wl.make_inputs(spec)
    xd, wd = x.to(dev), w.to(dev)
    pw = spa.prepare_weight(wd, spec.alpha, want_wt=name in DECODE)
    cfg = spa.PruneConfig(spec.n, spec.m, spec.score, spec.shift, spec.var_rescale, spec.act)
    fn = spa.sparse_linear_decode if name in DECODE else spa.sparse_linear_prefill
    y, idx, nu = fn(xd, pw, cfg, want_idx=True, want_nu=True)
    torch.cuda.synchronize()

    # every row: exactly n ascending positions inside each block
    kpos = idx.cpu().numpy().reshape(spec.t, spec.k // spec.m, spec.n).astype(np.int64)
    assert kpos.min() >= 0 and kpos.max() < spec.m
    if spec.n > 1:
        assert (np.diff(kpos, axis=-1) > 0).all(), "positions not strictly ascending within a block"

    # the oracle's prune: every token of a decode call, sampled rows of a
    # prefill (CLACT needs every token of the call for its column norm)
    rows = np.arange(spec.t) if name in DECODE else _sample(spec.t, 24, 1)
    f = None
    if spec.score == "weight":
        f = O.channel_factor(f32(w), spec.alpha)
        got_f = f32(pw.chan_scale)
        assert np.array_equal(got_f.view(np.uint32), f.view(np.uint32)), "weight factor differs from the oracle's"
    xs = f32(x) if spec.score == "clact" else f32(x[torch.as_tensor(rows)])
    pr = O.prune(xs, spec.dtype, spec.n, spec.m, score=spec.score, f=f, shift_mode=spec.shift,
                 var_rescale=spec.var_rescale, act=spec.act)
    if spec.score == "clact":
        pr = {key: (v[rows] if isinstance(v, np.ndarray) and v.ndim >= 1 and v.shape[0] == spec.t and key != "factor"
                    else v) for key, v in pr.items()}
    got_idx = idx.cpu().numpy()[rows]
    assert np.array_equal(got_idx, pr["idx"]), f"{name}: in-block positions differ on sampled rows"
    assert np.allclose(f32(nu)[rows], pr["nu"], rtol=1e-6, atol=0), f"{name}: nu differs"

    # every output of a decode call, sampled outputs of a prefill
    cols = np.arange(spec.n_out) if name in DECODE else _sample(spec.n_out, 96, 2)
    y_ref = O.linear(pr, f32(w[torch.as_tensor(cols)]))
    y_got = f32(y)[np.ix_(rows, cols)]
    err = O.rowwise_error(y_got, y_ref)
    assert err <= O.TOLERANCE[spec.dtype], f"{name}: sampled y error {err}"


@pytest.mark.parametrize("name", ["prefill", "relu2", "relu2_fused"])
def test_full_size_operand_as_timed(name):
    """The prompt workloads called as they are timed (no positions, no nu:
    the lean pruning pass): the 2:4 operand on every row holds two ascending
    in-block positions per block; on sampled rows the packed values, the
    positions and the shift equal the oracle's bit for bit; y on sampled rows
    x sampled columns."""
    assert torch.cuda.is_available(), "GPU tests need a device"
    dev = torch.device("cuda:0")
    spec = FULL[name]
    print(f"[full-size operand] {name}: t={spec.t} k={spec.k} n_out={spec.n_out}", flush=True)
    x, w = wl.make_inputs(spec)
    pw = spa.prepare_weight(w.to(dev), spec.alpha, want_wt=False)
    cfg = spa.PruneConfig(spec.n, spec.m, spec.score, spec.shift, spec.var_rescale, spec.act)
    ws = spa.workspace(2, spec.t, spec.k, spec.n_out, x.dtype, cfg, dev)
    y, idx, nu = spa.sparse_linear_prefill(x.to(dev), pw, cfg, ws=ws)
    torch.cuda.synchronize()
    assert idx is None and nu is None
    lay = spa.prefill_layout(spec.t, spec.k, x.dtype, cfg)
    vals, pos, _ = tiled_operand(ws, lay, spec.t, spec.k, False, spec.dtype)
    p2 = pos.reshape(spec.t, spec.k // 4, 2).astype(np.int64)
    assert p2.max() < 4 and (p2[..., 0] < p2[..., 1]).all(), "position words malformed"
    rows = _sample(spec.t, 24, 5)
    pr = O.prune(f32(x[torch.as_tensor(rows)]), spec.dtype, spec.n, spec.m, score=spec.score, shift_mode=spec.shift,
                 act=spec.act)
    assert np.array_equal(pos[rows], pr["idx"]), f"{name}: positions differ on sampled rows"
    assert np.array_equal(vals[rows], storage_bits(pr["vals"], spec.dtype)), f"{name}: packed values differ"
    eta = ws.cpu().numpy().view(np.uint8)[lay["eta"]:lay["eta"] + 4 * spec.t].view(np.float32)
    assert np.array_equal(eta[rows].view(np.uint32), pr["eta"].view(np.uint32)), f"{name}: shift differs"
    cols = _sample(spec.n_out, 96, 6)
    err = O.rowwise_error(f32(y)[np.ix_(rows, cols)], O.linear(pr, f32(w[torch.as_tensor(cols)])))
    assert err <= O.TOLERANCE[spec.dtype], f"{name}: sampled y error {err}"


@pytest.mark.parametrize("fmt,n,m,t,k", [("comb", 2, 4, 4096, 16384), ("bitmap", 2, 4, 4096, 16384),
                                         ("comb", 16, 32, 32, 14336), ("comb", 8, 16, 1, 4096)])
def test_meta_full_size(fmt, n, m, t, k):
    # every row: decode(encode(positions)) gives the positions back; sampled
    # rows: the codes equal the oracle's bit for bit
    assert torch.cuda.is_available(), "GPU tests need a device"
    dev = torch.device("cuda:0")
    print(f"[full-size meta] {fmt} {n}:{m} t={t} k={k}", flush=True)
    idx = wl.random_positions(t, k, n, m, seed=3)
    idx_d = idx.to(dev)
    codes = spa.encode_meta(idx_d, n, m, fmt)
    back = spa.decode_meta(codes, k, n, m, fmt)
    torch.cuda.synchronize()
    assert torch.equal(back, idx_d), "round trip differs"
    rows = _sample(t, 12, 4)
    want = O.encode_meta(idx.numpy()[rows], n, m, fmt)
    assert np.array_equal(codes.cpu().numpy().view(np.uint32)[rows], want)


def test_amber_full_size():
    # the Amber-Pruner factor of the decode layer's weight [14336, 4096] bf16:
    # the global percentiles, mean and variance over all 58.7 M weights; the
    # per-channel sums on sampled channels
    assert torch.cuda.is_available(), "GPU tests need a device"
    dev = torch.device("cuda:0")
    spec = wl.SPECS["decode"]
    print(f"[full-size amber] n_out={spec.n_out} k={spec.k}", flush=True)
    _, w = wl.make_inputs(spec)
    got = f32(spa.prepare_amber(w.to(dev), 1.0))
    torch.cuda.synchronize()
    cols = _sample(spec.k, 32, 5)
    want = O.amber_factor(f32(w), 1.0, cols=cols)
    assert np.allclose(got[cols], want, rtol=1e-6, atol=0), np.abs(got[cols] / want - 1).max()


# ---------------------------------------------------------------------------
# maximum sizes
# ---------------------------------------------------------------------------
def test_max_prune_row():
    # one token row of 2^24 channels, the largest k the library takes
    assert torch.cuda.is_available(), "GPU tests need a device"
    dev = torch.device("cuda:0")
    spec = wl.SPECS["prefill"].with_(t=2, k=1 << 24, n_outliers=0, shift="token_mean")
    print(f"[max size] prune_nm t={spec.t} k={spec.k}", flush=True)
    x, _ = wl.make_inputs(spec, with_weight=False)
    vals, idx, eta, nu = spa.prune_nm(x.to(dev), spa.PruneConfig(2, 4, "magnitude", "token_mean"))
    torch.cuda.synchronize()
    pr = O.prune(f32(x), "bf16", 2, 4, shift_mode="token_mean")
    assert np.array_equal(f32(eta).view(np.uint32), pr["eta"].view(np.uint32))
    assert np.array_equal(idx.cpu().numpy(), pr["idx"])
    assert np.array_equal(vals.cpu().view(torch.int16).numpy(),
                          torch.from_numpy(pr["vals"]).to(torch.bfloat16).view(torch.int16).numpy())


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_max_prefill_k(n, m):
    # k = 2^23, the largest the prefill GEMMs take (a 256-row weight tile is
    # then just under 4 GiB of 32-bit offsets)
    assert torch.cuda.is_available(), "GPU tests need a device"
    dev = torch.device("cuda:0")
    spec = wl.SPECS["prefill"].with_(t=3, k=1 << 23, n_out=256, n=n, m=m, n_outliers=0)
    print(f"[max size] prefill t={spec.t} k={spec.k} n_out={spec.n_out} {n}:{m}", flush=True)
    x, w = wl.make_inputs(spec)
    pw = spa.prepare_weight(w.to(dev), 0.0, want_wt=False)
    y, idx, nu = spa.sparse_linear_prefill(x.to(dev), pw, spa.PruneConfig(n, m, "magnitude", "token_mean"),
                                           want_idx=True, want_nu=True)
    torch.cuda.synchronize()
    pr = O.prune(f32(x), "bf16", n, m, shift_mode="token_mean")
    assert np.array_equal(idx.cpu().numpy(), pr["idx"])
    cols = _sample(spec.n_out, 16, 7)                       # includes the last weight row (the largest offset)
    wc = w[torch.as_tensor(cols)]
    y_ref = O.linear(pr, f32(wc))
    err = O.rowwise_error(f32(y)[:, cols], y_ref)
    assert err <= O.TOLERANCE["bf16"], err


@pytest.mark.parametrize("k", [262080, 262144])
def test_max_decode_weight(k):
    # one token, 4096 outputs: k = 262080 keeps the channel-major weight just
    # under 2 GiB (the wide one-token kernel's 32-bit offsets); k = 262144 is
    # exactly 2 GiB and takes the fused kernel, whose per-split row list then
    # needs two passes of the workgroup's threads
    assert torch.cuda.is_available(), "GPU tests need a device"
    dev = torch.device("cuda:0")
    spec = wl.SPECS["decode"].with_(t=1, k=k, n_out=4096, score="magnitude", shift="none", n_outliers=0)
    print(f"[max size] decode t=1 k={k} n_out=4096 ({k * 4096 * 2} B of weight)", flush=True)
    x, w = wl.make_inputs(spec)
    pw = spa.prepare_weight(w.to(dev), 0.0)
    y, idx, nu = spa.sparse_linear_decode(x.to(dev), pw, spa.PruneConfig(8, 16), want_idx=True)
    torch.cuda.synchronize()
    del pw
    pr = O.prune(f32(x), "bf16", 8, 16)
    assert np.array_equal(idx.cpu().numpy(), pr["idx"])
    cols = _sample(4096, 96, 6)
    y_ref = O.linear(pr, f32(w[torch.as_tensor(cols)]), s=np.zeros(cols.size))
    err = O.rowwise_error(f32(y)[:, cols], y_ref)
    assert err <= O.TOLERANCE["bf16"], err


def test_ffn_relu2_full_size():
    # the squared-ReLU FFN at the relu2 layer's sizes: x [4096, 4096], up
    # [16384, 4096], down [4096, 16384], bf16.  Every row's positions against
    # the oracle's pruning of the GPU's own up-projection (the library's dense
    # GEMM: same main loop and rounding); y on sampled rows and columns
    assert torch.cuda.is_available(), "GPU tests need a device"
    dev = torch.device("cuda:0")
    t, hidden, ffn, n_out = 4096, 4096, 16384, 4096
    print(f"[full-size ffn] t={t} hidden={hidden} ffn={ffn} n_out={n_out}", flush=True)
    spec = wl.SPECS["prefill"].with_(t=t, k=hidden, n_out=ffn, n_outliers=0)
    x, w_up = wl.make_inputs(spec)
    _, w_dn = wl.make_inputs(spec.with_(k=ffn, n_out=n_out), seed=1)
    xd, upd = x.to(dev), w_up.to(dev)
    y, idx = spa.sparse_ffn_relu2_prefill(xd, upd, w_dn.to(dev), want_idx=True)
    u, _, _ = spa.sparse_linear_prefill(xd, spa.PreparedWeight(upd, None, None, None), spa.PruneConfig(4, 4))
    torch.cuda.synchronize()
    u_cpu = f32(u)
    del u
    pr_all = O.prune(u_cpu, "bf16", 2, 4, act="relu2")
    assert np.array_equal(idx.cpu().numpy(), pr_all["idx"]), "fused FFN positions differ"
    rows = _sample(t, 16, 8)
    cols = _sample(n_out, 64, 9)
    pr = O.ffn_relu2(f32(x[torch.as_tensor(rows)]), f32(w_up), f32(w_dn[torch.as_tensor(cols)]), "bf16")
    err = O.rowwise_error(f32(y)[np.ix_(rows, cols)], pr["y"])
    assert err <= O.TOLERANCE["bf16"], err

"""GPU parity: the HIP library against the CPU oracle, element by element.

Masks (in-block positions), packed values and the per-token shift must
match bit for bit; the output y within the row-normwise tolerance (2e-2 for
16-bit storage, 1e-5 for float32); nu within 1e-6 relative.  Inputs are the
seeded workloads; the oracle never sees anything the GPU computed.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import nm_oracle as O
from gpu_util import TORCH_DT, f32, oracle_for, storage_bits, tensor_bits, tiled_operand

pytestmark = pytest.mark.gpu

spa = pytest.importorskip("activation_sparsification_amd")


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a device"
    return torch.device("cuda:0")


def _cfg(spec, n=None, m=None):
    return spa.PruneConfig(n or spec.n, m or spec.m, spec.score, spec.shift, spec.var_rescale, spec.act)


def _check_prune(pr, vals, idx, eta, nu, dtype):
    assert np.array_equal(tensor_bits(vals), storage_bits(pr["vals"], dtype)), "packed values differ"
    assert np.array_equal(idx.cpu().numpy(), pr["idx"]), "in-block positions differ"
    assert np.array_equal(f32(eta).view(np.uint32), pr["eta"].view(np.uint32)), "eta differs"
    assert np.allclose(f32(nu), pr["nu"], rtol=1e-6, atol=0), "nu differs"


# ---------------------------------------------------------------------------
# prepare_weight
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "decode_small", "batched_small_t8"])
@pytest.mark.parametrize("alpha", [0.0, 0.5, 1.0])
def test_prepare_weight(name, alpha):
    spec = {s.name: s for s in wl.parity_specs()}[name]
    _, w = wl.make_inputs(spec)
    dev = _dev()
    pw = spa.prepare_weight(w.to(dev), alpha)
    torch.cuda.synchronize()
    assert torch.equal(pw.wt.cpu(), w.t().contiguous())
    f = O.channel_factor(f32(w), alpha)
    got = f32(pw.chan_scale)
    assert np.array_equal(got.view(np.uint32), f.view(np.uint32)), (np.abs(got - f) / f).max()
    s = O.row_sum(f32(w)).astype(np.float32)
    assert np.array_equal(f32(pw.row_sum), s)


# ---------------------------------------------------------------------------
# squared-ReLU FFN (up-projection epilogue prunes and packs)
# ---------------------------------------------------------------------------
FFN_CASES = [("bf16", 200, 512, 1024, 264), ("f16", 77, 320, 320, 136), ("bf16", 300, 256, 640, 520),
             ("bf16", 1, 64, 64, 8), ("f16", 513, 128, 192, 40), ("bf16", 33, 128, 256, 37)]


def _ffn_inputs(dtype, t, hidden, ffn, n_out, seed):
    spec = wl.SPECS["prefill"].with_(t=t, k=hidden, n_out=ffn, dtype=dtype, n_outliers=0)
    x, w_up = wl.make_inputs(spec, seed=seed)
    _, w_dn = wl.make_inputs(spec.with_(k=ffn, n_out=n_out), seed=seed + 1)
    return x, w_up, w_dn


def ffn_up_reference(x, w_up, dev):
    """u = x W_up^T from the library's dense GEMM (a 4:4 prefill keeps every
    channel): the same matrix-core main loop and rounding as the fused
    up-projection, whose epilogue squares and prunes this u."""
    pw = spa.PreparedWeight(w_up, None, None, None)
    u, _, _ = spa.sparse_linear_prefill(x, pw, spa.PruneConfig(4, 4))
    return u


@pytest.mark.parametrize("dtype,t,hidden,ffn,n_out", FFN_CASES)
def test_ffn_relu2(dtype, t, hidden, ffn, n_out):
    dev = _dev()
    x, w_up, w_dn = _ffn_inputs(dtype, t, hidden, ffn, n_out, seed=t)
    xd, upd = x.to(dev), w_up.to(dev)
    nb = spa.lib().spa_ffn_workspace_bytes(t, ffn, spa._binding.DTYPE[x.dtype])
    y, idx = spa.sparse_ffn_relu2_prefill(xd, upd, w_dn.to(dev), want_idx=True)
    u = ffn_up_reference(xd, upd, dev)
    torch.cuda.synchronize()
    ws = spa._binding._WS_CACHE[(str(dev), "ffn", nb)]
    # the oracle prunes the squared ReLU of the GPU's own u: positions and the
    # packed operand of the down-projection bit for bit
    pr = O.prune(f32(u), dtype, 2, 4, act="relu2")
    assert np.array_equal(idx.cpu().numpy(), pr["idx"]), "fused FFN positions differ"
    t_pad = (t + 255) // 256 * 256
    lay = {"vals": 0, "meta": (t_pad * ffn + 255) // 256 * 256, "t_pad": t_pad}
    vals, pos, _ = tiled_operand(ws, lay, t, ffn, False, dtype)
    assert np.array_equal(vals, storage_bits(pr["vals"], dtype)), "fused FFN packed operand differs"
    assert np.array_equal(pos, pr["idx"])
    # y against the float64 oracle of the whole FFN, and against the oracle's
    # down-projection of the GPU's activation
    ref = O.ffn_relu2(f32(x), f32(w_up), f32(w_dn), dtype)
    assert O.rowwise_error(f32(y), ref["y"]) <= O.TOLERANCE[dtype]
    err = O.rowwise_error(f32(y), O.linear(pr, f32(w_dn), s=np.zeros(n_out)))
    assert err <= O.TOLERANCE[dtype], err


def test_ffn_relu2_invalid():
    dev = _dev()
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(spa.SpaError):       # ffn not a multiple of 64
        spa.sparse_ffn_relu2_prefill(x, torch.zeros((96, 64), dtype=torch.bfloat16, device=dev),
                                     torch.zeros((8, 96), dtype=torch.bfloat16, device=dev))
    with pytest.raises(spa.SpaError):       # float32
        spa.sparse_ffn_relu2_prefill(x.float(), torch.zeros((64, 64), device=dev), torch.zeros((8, 64), device=dev))


# ---------------------------------------------------------------------------
# running-average variance factor (var_rescale = 2)
# ---------------------------------------------------------------------------
EMA_CASES = [
    ("prune_bf16_2_4", "prune", wl.SPECS["prefill"].with_(t=37, k=1024, n_outliers=0)),
    ("prune_f32_16_32", "prune", wl.SPECS["batched"].with_(t=5, k=512, dtype="f32")),
    ("prefill_2_4", "prefill", wl.SPECS["prefill"].with_(t=300, k=512, n_out=272, n_outliers=0)),
    ("prefill_8_16", "prefill", wl.SPECS["prefill"].with_(t=77, k=320, n_out=300, n=8, m=16, n_outliers=0)),
    ("decode_t1_wide", "decode", wl.SPECS["decode"].with_(t=1, k=2048, n_out=4096)),
    ("decode_t1_narrow", "decode", wl.SPECS["batched"].with_(t=1, k=1024, n_out=776)),
    ("decode_t3", "decode", wl.SPECS["batched"].with_(t=3, k=512, n_out=136)),
    ("decode_mm_t20", "decode", wl.SPECS["batched"].with_(t=20, k=1056, n_out=328)),
    ("decode_f32_t8", "decode", wl.SPECS["tiny"].with_(t=8)),
]


@pytest.mark.parametrize("label,entry,spec", EMA_CASES, ids=[c[0] for c in EMA_CASES])
def test_var_running_average(label, entry, spec):
    dev = _dev()
    spec = spec.with_(var_rescale=2)
    x, w = wl.make_inputs(spec)
    r_in = (np.random.Generator(np.random.PCG64(spec.t)).uniform(0.05, 2.0, size=spec.t)).astype(np.float32)
    st_in = torch.from_numpy(r_in).to(dev)
    st_out = torch.full((spec.t,), -1.0, dtype=torch.float32, device=dev)
    cfg = spa.PruneConfig(spec.n, spec.m, spec.score, spec.shift, 2, spec.act, st_in, st_out)
    f = None
    if entry == "prune":
        f = O.channel_factor(f32(w), spec.alpha) if spec.score == "weight" else None
        vals, idx, eta, nu = spa.prune_nm(x.to(dev), cfg, chan_scale=None if f is None else torch.from_numpy(f).to(dev))
    else:
        pw = spa.prepare_weight(w.to(dev), spec.alpha, want_wt=entry == "decode")
        f = O.channel_factor(f32(w), spec.alpha) if spec.score == "weight" else None
        if f is not None:
            assert np.array_equal(f32(pw.chan_scale).view(np.uint32), f.view(np.uint32))
        fn = spa.sparse_linear_decode if entry == "decode" else spa.sparse_linear_prefill
        y, idx, nu = fn(x.to(dev), pw, cfg, want_idx=True, want_nu=True)
    torch.cuda.synchronize()
    pr = O.prune(f32(x), spec.dtype, spec.n, spec.m, score=spec.score, f=f, shift_mode=spec.shift, var_rescale=2,
                 var_state=r_in)
    assert np.array_equal(idx.cpu().numpy(), pr["idx"])
    assert np.allclose(f32(nu), pr["nu"], rtol=1e-6, atol=0), np.abs(f32(nu) / pr["nu"] - 1).max()
    assert np.allclose(f32(st_out), pr["var_state"], rtol=1e-6, atol=0)
    assert np.array_equal(f32(st_in), r_in)                            # the input state is left alone
    if entry != "prune":
        err = O.rowwise_error(f32(y), O.linear(pr, f32(w)))
        assert err <= O.TOLERANCE[spec.dtype], err


# ---------------------------------------------------------------------------
# static shift table (S-PTS)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_eta_table(dtype):
    # three calibration batches, ids repeating across them, unseen ids and ids
    # outside the table; the table's float64 sums are atomic, so an entry may
    # differ from the oracle's in its last float32 unit
    dev = _dev()
    vocab = 50
    cal = spa.EtaCalibration(vocab, dev)
    batches = []
    for b, (t, k) in enumerate([(37, 512), (64, 512), (5, 512)]):
        spec = wl.SPECS["decode"].with_(t=t, k=k, dtype=dtype, n_outliers=0)
        x, _ = wl.make_inputs(spec, seed=b, with_weight=False)
        ids = np.random.Generator(np.random.PCG64(100 + b)).integers(-3, vocab + 3, size=t)
        cal.add(x.to(dev), torch.from_numpy(ids))
        batches.append((f32(x), ids))
    got = f32(cal.table())
    torch.cuda.synchronize()
    # the oracle collects only ids inside the table
    inside = [(x[(i >= 0) & (i < vocab)], i[(i >= 0) & (i < vocab)]) for x, i in batches]
    want = O.eta_table(inside, vocab)
    ulp = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1, ulp.max()
    assert (got[want == 0] == 0).all()
    # lookup: bit for bit on the oracle's table
    ids = torch.tensor([3, -1, 49, 50, 0, 7, 7], dtype=torch.int32)
    eta = spa.eta_lookup(torch.from_numpy(want).to(dev), ids)
    torch.cuda.synchronize()
    assert np.array_equal(f32(eta), O.eta_lookup(want, ids.numpy()))


def test_static_shift_drives_decode():
    # S-PTS end to end: the looked-up shift as eta_in of a decode call
    dev = _dev()
    spec = wl.SPECS["decode"].with_(t=3, k=1024, n_out=776, shift="given")
    x, w = wl.make_inputs(spec)
    table = (np.arange(20, dtype=np.float32) - 10) / 64
    ids = np.array([4, 19, 11])
    eta = spa.eta_lookup(torch.from_numpy(table).to(dev), torch.from_numpy(ids))
    pw = spa.prepare_weight(w.to(dev), spec.alpha)
    y, idx, nu = spa.sparse_linear_decode(x.to(dev), pw, _cfg(spec), eta_in=eta, want_idx=True, want_nu=True)
    torch.cuda.synchronize()
    f = O.channel_factor(f32(w), spec.alpha)
    assert np.array_equal(f32(pw.chan_scale).view(np.uint32), f.view(np.uint32))
    pr = oracle_for(spec, x, w, f=f, eta_in=torch.from_numpy(O.eta_lookup(table, ids)))
    assert np.array_equal(idx.cpu().numpy(), pr["idx"])
    assert O.rowwise_error(f32(y), pr["y"]) <= O.TOLERANCE[spec.dtype]


# ---------------------------------------------------------------------------
# prepare_amber
# ---------------------------------------------------------------------------
def _amber_weights(kind, dtype, n_out, k, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.normal(0.0, 0.02, size=(n_out, k))
    if kind == "outliers":                                   # a few planted outliers, both signs
        idx = rng.integers(0, n_out * k, size=max(4, n_out * k // 300))
        w.ravel()[idx] = rng.choice([-1.0, 1.0], size=idx.size) * rng.uniform(0.2, 2.0, size=idx.size)
    elif kind == "shifted":                                  # non-zero mean
        w = w + 0.3
    elif kind == "levels":                                   # many equal values around the percentiles
        w = np.round(w * 200) / 200
    return torch.from_numpy(w.astype(np.float32)).to(TORCH_DT[dtype])


AMBER_CASES = [(kind, dt, n_out, k) for kind in ["normal", "outliers", "shifted", "levels"]
               for dt in ["bf16", "f16", "f32"] for n_out, k in [(300, 77), (1000, 1024)]]
AMBER_CASES.append(("normal", "bf16", 1, 16))


@pytest.mark.parametrize("kind,dtype,n_out,k", AMBER_CASES)
@pytest.mark.parametrize("alpha", [1.0, 0.5])
def test_prepare_amber(kind, dtype, n_out, k, alpha):
    dev = _dev()
    w = _amber_weights(kind, dtype, n_out, k, seed=n_out + k)
    got = f32(spa.prepare_amber(w.to(dev), alpha))
    torch.cuda.synchronize()
    want = O.amber_factor(f32(w), alpha)
    assert np.allclose(got, want, rtol=1e-6, atol=0), np.abs(got / want - 1).max()


def test_amber_factor_drives_the_masks():
    # the weight-aware score with the Amber factor (the oracle's float32
    # vector feeds both sides)
    dev = _dev()
    spec = wl.SPECS["decode"].with_(t=5, k=1024, n_out=512)
    x, w = wl.make_inputs(spec)
    f = O.amber_factor(f32(w), 1.0)
    pr = O.prune(f32(x), spec.dtype, spec.n, spec.m, score="weight", f=f, shift_mode=spec.shift)
    vals, idx, eta, nu = spa.prune_nm(x.to(dev), _cfg(spec), chan_scale=torch.from_numpy(f).to(dev))
    torch.cuda.synchronize()
    _check_prune(pr, vals, idx, eta, nu, spec.dtype)


# ---------------------------------------------------------------------------
# prune_nm
# ---------------------------------------------------------------------------
PRUNE_CASES = []
for s in wl.parity_specs():
    PRUNE_CASES.append((s.name, s))
for dt in ["bf16", "f16", "f32"]:
    for n, m in [(1, 4), (2, 4), (3, 8), (4, 8), (8, 16), (5, 16), (16, 32), (8, 32), (32, 32)]:
        for score, shift, var in [("magnitude", "none", False), ("weight", "token_mean", True),
                                  ("clact", "given", True)]:
            base = wl.SPECS["decode"].with_(name="sweep", t=3, k=256, n_out=64, dtype=dt, n=n, m=m, score=score,
                                            shift=shift, var_rescale=var, alpha=0.5)
            PRUNE_CASES.append((f"{dt}-{n}:{m}-{score}-{shift}-{int(var)}", base))
# the squared-ReLU input transform: every dtype, the shift and CLACT kernels that
# read the input themselves, and a row longer than one pass (k > 256 x 16)
for dt in ["bf16", "f16", "f32"]:
    for n, m in [(2, 4), (8, 16), (16, 32)]:
        for score, shift, var, xd in [("magnitude", "token_mean", True, "normal"),
                                      ("clact", "token_mean", False, "preact_shifted"),
                                      ("weight", "none", False, "normal")]:
            base = wl.SPECS["decode"].with_(name="sweep_act", t=3, k=256, n_out=64, dtype=dt, n=n, m=m, score=score,
                                            shift=shift, var_rescale=var, alpha=0.5, act="relu2", x_dist=xd,
                                            n_outliers=0)
            PRUNE_CASES.append((f"act-{dt}-{n}:{m}-{score}-{shift}-{int(var)}", base))
PRUNE_CASES.append(("act-long-row", wl.SPECS["relu2_fused"].with_(t=3, k=8192, shift="token_mean")))


@pytest.mark.parametrize("label,spec", PRUNE_CASES, ids=[c[0] for c in PRUNE_CASES])
def test_prune_parity(label, spec):
    dev = _dev()
    x, w = wl.make_inputs(spec)
    eta_in = wl.make_eta(spec.t, 3) if spec.shift == "given" else None
    f = O.channel_factor(f32(w), spec.alpha) if spec.score == "weight" else None
    pr = oracle_for(spec, x, None, f=f, eta_in=eta_in)
    vals, idx, eta, nu = spa.prune_nm(x.to(dev), _cfg(spec),
                                      chan_scale=None if f is None else torch.from_numpy(f).to(dev),
                                      eta_in=None if eta_in is None else eta_in.to(dev))
    torch.cuda.synchronize()
    _check_prune(pr, vals, idx, eta, nu, spec.dtype)


ADV_KINDS = ["equal", "zeros", "signed_pairs", "signed_zero", "one_big", "few_levels"]


@pytest.mark.parametrize("kind", ADV_KINDS)
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (8, 16), (16, 32), (1, 32)])
def test_prune_ties(kind, n, m):
    dev = _dev()
    spec = wl.SPECS["relu2"].with_(t=5, k=512, n=n, m=m, dtype="bf16")
    x = wl.adversarial_x(kind, spec.t, spec.k, m, "bf16", seed=n + m)
    pr = oracle_for(spec, x, None)
    vals, idx, eta, nu = spa.prune_nm(x.to(dev), _cfg(spec))
    torch.cuda.synchronize()
    _check_prune(pr, vals, idx, eta, nu, "bf16")


def test_prune_empty_and_invalid():
    dev = _dev()
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    vals, idx, eta, nu = spa.prune_nm(x, spa.PruneConfig(2, 4))
    assert vals.shape == (0, 32)
    with pytest.raises(spa.SpaError):
        spa.prune_nm(torch.zeros((2, 60), dtype=torch.bfloat16, device=dev), spa.PruneConfig(2, 4))
    with pytest.raises(spa.SpaError):
        spa.prune_nm(torch.zeros((2, 64), dtype=torch.bfloat16, device=dev), spa.PruneConfig(5, 4))


# ---------------------------------------------------------------------------
# compact block metadata
# ---------------------------------------------------------------------------
META_CASES = []
for fmt in ["comb", "bitmap"]:
    for n, m in [(2, 4), (1, 4), (3, 4), (4, 4), (4, 8), (3, 8), (8, 16), (5, 16), (16, 32), (12, 32), (1, 32),
                 (32, 32)]:
        META_CASES.append((fmt, n, m, 300))
    # several workgroups per row, rows that start off 16-byte boundaries
    for n, m in [(2, 4), (1, 4), (8, 16), (16, 32), (3, 8)]:
        META_CASES.append((fmt, n, m, 5001))
# 2:4 codes and masks of rows that fill whole words (blocks per row a multiple
# of 32, of 8 for masks): one flat stream over all rows; one partial
# workgroup, and two workgroups whose later pieces run past the end
META_CASES += [("comb", 2, 4, 96), ("comb", 2, 4, 4128), ("bitmap", 2, 4, 40), ("bitmap", 2, 4, 4104)]


@pytest.mark.parametrize("fmt,n,m,nb", META_CASES)
def test_meta_parity(fmt, n, m, nb):
    # rows of 300 blocks: several waves, a partial workgroup, a ragged last word
    dev = _dev()
    t, k = 3, nb * m
    idx = wl.random_positions(t, k, n, m, seed=n * 64 + m)
    want = O.encode_meta(idx.numpy(), n, m, fmt)
    codes = spa.encode_meta(idx.to(dev), n, m, fmt)
    back = spa.decode_meta(codes, k, n, m, fmt)
    torch.cuda.synchronize()
    got = codes.cpu().numpy().view(np.uint32)
    assert got.shape == want.shape
    assert np.array_equal(got, want), "codes differ"
    assert np.array_equal(back.cpu().numpy(), idx.numpy()), "decoded positions differ"
    # the oracle's codes decode to the same positions on the GPU
    back2 = spa.decode_meta(torch.from_numpy(want.view(np.int32)).to(dev), k, n, m, fmt)
    torch.cuda.synchronize()
    assert np.array_equal(back2.cpu().numpy(), idx.numpy())


@pytest.mark.parametrize("fmt", ["comb", "bitmap"])
def test_meta_of_pruned_masks(fmt):
    # the positions prune_nm returns, packed and unpacked
    dev = _dev()
    spec = wl.SPECS["relu2"].with_(t=7, k=4096 + 64)
    x, _ = wl.make_inputs(spec, with_weight=False)
    pr = oracle_for(spec, x, None)
    codes = spa.encode_meta(torch.from_numpy(pr["idx"]).to(dev), 2, 4, fmt)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy().view(np.uint32), O.encode_meta(pr["idx"], 2, 4, fmt))


def test_meta_empty_and_invalid():
    dev = _dev()
    idx = torch.zeros((0, 32), dtype=torch.uint8, device=dev)
    assert spa.encode_meta(idx, 2, 4).shape == (0, 2)                  # 16 blocks x 3 bits -> 2 words
    with pytest.raises(spa.SpaError):
        spa.encode_meta(torch.zeros((2, 30), dtype=torch.uint8, device=dev), 2, 6)   # m = 6 is not a width
    with pytest.raises(spa.SpaError):
        spa.decode_meta(torch.zeros((2, 3), dtype=torch.int32, device=dev), 64, 5, 4)  # n > m


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
DECODE_CASES = [s for s in wl.parity_specs() if s.t <= 32]
for t in [1, 2, 3, 4, 5, 8, 13, 16, 17, 32]:
    DECODE_CASES.append(wl.SPECS["decode"].with_(name=f"decode_t{t}", t=t, k=1024, n_out=776))
for dt in ["bf16", "f16"]:
    for n, m in [(2, 4), (4, 8), (8, 16), (16, 32), (16, 16)]:
        DECODE_CASES.append(wl.SPECS["batched"].with_(name=f"dec_{dt}_{n}_{m}_t3", t=3, k=512, n_out=136, dtype=dt,
                                                      n=n, m=m))
        DECODE_CASES.append(wl.SPECS["batched"].with_(name=f"dec_{dt}_{n}_{m}_t20", t=20, k=512, n_out=136,
                                                      dtype=dt, n=n, m=m, score="magnitude", shift="token_mean",
                                                      var_rescale=False))
DECODE_CASES.append(wl.SPECS["tiny"].with_(name="tiny_f32_t8", t=8, shift="token_mean"))
# one token, outputs of at least eight 512-column tiles (the wide one-token kernel):
# a ragged last tile, a channel split whose last wave is partial, more kept rows
# per wave than one batch of loads (3:4), several channel rounds per workgroup,
# every block width, both 16-bit types and every score and shift
T1_WIDE = [
    ("t1w_ragged_tile", dict(k=4096, n_out=4104)),
    ("t1w_partial_wave", dict(k=1040, n_out=4096)),
    ("t1w_3of4", dict(k=8192, n_out=4096, n=3, m=4, score="magnitude")),
    ("t1w_rounds", dict(k=32768, n_out=4096, shift="none")),
    ("t1w_1of8_given", dict(k=2048, n_out=4608, n=1, m=8, shift="given")),
    ("t1w_f16_clact_var", dict(k=2048, n_out=4096, n=16, m=32, dtype="f16", score="clact", shift="none",
                               var_rescale=True)),
    ("t1w_f16_2of4_var", dict(k=1024, n_out=5120, n=2, m=4, dtype="f16", score="magnitude", var_rescale=True)),
]
for nm, kw in T1_WIDE:
    DECODE_CASES.append(wl.SPECS["decode"].with_(name=nm, t=1, **kw))
# matrix-core path: fewer 64-channel steps than one ring stage, a ragged last step
# (k % 64 = 16), a ragged pruning chunk (k % 256 != 0), and a ragged row tile
DECODE_CASES.append(wl.SPECS["batched"].with_(name="mm_two_steps", t=8, k=128, n_out=200))
DECODE_CASES.append(wl.SPECS["batched"].with_(name="mm_ragged_step", t=24, k=1040, n_out=328, n=8, m=16))
DECODE_CASES.append(wl.SPECS["batched"].with_(name="mm_bf16_weight_mean", t=12, k=1600, n_out=264, dtype="bf16",
                                              n=2, m=4, score="weight", alpha=0.5, shift="token_mean",
                                              var_rescale=True))
DECODE_CASES.append(wl.SPECS["decode"].with_(name="decode_given_shift", t=2, k=512, n_out=256, shift="given"))
# the fused kernel with more m-blocks per channel split than threads (its row
# list is built over two passes): float32 one token, a narrow 16-bit output,
# and two tokens with one split per column tile
DECODE_CASES.append(wl.SPECS["decode"].with_(name="fused_t1_f32_two_passes", t=1, k=32768, n_out=4096, dtype="f32"))
DECODE_CASES.append(wl.SPECS["decode"].with_(name="fused_t1_bf16_2of4_two_passes", t=1, k=32768, n_out=2048, n=2,
                                             m=4))
DECODE_CASES.append(wl.SPECS["decode"].with_(name="fused_f32_t2_two_passes", t=2, k=8192, n_out=12288, dtype="f32"))
# two to four 16-bit tokens take the matrix-core path: wide and narrow outputs,
# ragged tiles and a k that ends inside a 64-channel step
DECODE_CASES.append(wl.SPECS["decode"].with_(name="mm_t2_wide", t=2, k=8192, n_out=12288))
DECODE_CASES.append(wl.SPECS["batched"].with_(name="mm_t2_clact_var", t=2, k=2080, n_out=520))
DECODE_CASES.append(wl.SPECS["decode"].with_(name="mm_t4_given", t=4, k=1040, n_out=200, shift="given"))
# the token mean on the matrix-core path: formed inside the pruning pass up to
# t k = 65536 (the limit itself here), by a pass of its own beyond it
DECODE_CASES.append(wl.SPECS["decode"].with_(name="mm_t16_mean_in_pass_at_limit", t=16, k=4096, n_out=264))
DECODE_CASES.append(wl.SPECS["decode"].with_(name="mm_t8_mean_pass_long_rows", t=8, k=16384, n_out=264))
DECODE_CASES.append(wl.SPECS["decode"].with_(name="mm_t3_mean_pass_relu2", t=3, k=32768, n_out=136, act="relu2",
                                             x_dist="normal", n_outliers=0))
# float32 with 2 and 3 tokens (the fused kernel's multi-token forms)
DECODE_CASES.append(wl.SPECS["decode"].with_(name="fused_f32_t2", t=2, k=1024, n_out=776, dtype="f32"))
DECODE_CASES.append(wl.SPECS["batched"].with_(name="fused_f32_t3_clact_var", t=3, k=512, n_out=136, dtype="f32"))
# the squared-ReLU input transform on every decode kernel: one token (wide and
# narrow outputs), 2-4 tokens, float32, and the matrix-core path
ACT = dict(act="relu2", x_dist="normal", n_outliers=0)
DECODE_CASES.append(wl.SPECS["decode"].with_(name="act_t1w", t=1, k=4096, n_out=4096, **ACT))
DECODE_CASES.append(wl.SPECS["decode"].with_(name="act_t1w_preact", t=1, k=2048, n_out=4608,
                                             **dict(ACT, x_dist="preact_shifted")))
DECODE_CASES.append(wl.SPECS["decode"].with_(name="act_t1_narrow", t=1, k=1024, n_out=776, **ACT))
DECODE_CASES.append(wl.SPECS["batched"].with_(name="act_fused_t3_clact", t=3, k=512, n_out=136, **ACT))
DECODE_CASES.append(wl.SPECS["decode"].with_(name="act_fused_t4_mean", t=4, k=1024, n_out=776, **ACT))
DECODE_CASES.append(wl.SPECS["tiny"].with_(name="act_tiny_f32_t8", t=8, shift="token_mean", act="relu2"))
DECODE_CASES.append(wl.SPECS["batched"].with_(name="act_mm_t20_clact", t=20, k=1056, n_out=328, **ACT))
DECODE_CASES.append(wl.SPECS["batched"].with_(name="act_mm_t12_bf16_mean", t=12, k=1600, n_out=264, dtype="bf16",
                                              n=2, m=4, score="weight", alpha=0.5, shift="token_mean",
                                              var_rescale=True, **ACT))


@pytest.mark.parametrize("spec", DECODE_CASES, ids=[s.name for s in DECODE_CASES])
def test_decode_parity(spec):
    dev = _dev()
    x, w = wl.make_inputs(spec)
    eta_in = wl.make_eta(spec.t, 5) if spec.shift == "given" else None
    pw = spa.prepare_weight(w.to(dev), spec.alpha)
    f = f32(pw.chan_scale) if spec.score == "weight" else None
    if f is not None:
        assert np.array_equal(f.view(np.uint32), O.channel_factor(f32(w), spec.alpha).view(np.uint32))
    pr = oracle_for(spec, x, w, f=f, eta_in=eta_in)
    y, idx, nu = spa.sparse_linear_decode(x.to(dev), pw, _cfg(spec),
                                          eta_in=None if eta_in is None else eta_in.to(dev), want_idx=True,
                                          want_nu=True)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), pr["idx"]), "decode masks differ"
    assert np.allclose(f32(nu), pr["nu"], rtol=1e-6, atol=0)
    err = O.rowwise_error(f32(y), pr["y"])
    assert err <= O.TOLERANCE[spec.dtype], err


# Tie-heavy tokens through each decode kernel: the one-token kernel (rank by
# lane swizzles; n_out >= 4096), the fused 2-4 token kernel (selection
# network) and the matrix-core path's pruning pass (64-bit rank keys).  Ties
# go to the lower position, as in the oracle.
DECODE_TIE_CASES = [("t1_8_16", 1, 8, 16, 4096, "bf16", "none"), ("t1_16_32", 1, 16, 32, 4096, "f16", "token_mean"),
                    ("fused_t3_8_16", 3, 8, 16, 264, "bf16", "none"), ("mm_t8_16_32", 8, 16, 32, 256, "f16", "none"),
                    ("mm_t20_2_4", 20, 2, 4, 256, "bf16", "token_mean"), ("mm_t6_1_4", 6, 1, 4, 200, "f16", "none")]


@pytest.mark.parametrize("kind", ["equal", "zeros", "signed_pairs", "one_big", "few_levels"])
@pytest.mark.parametrize("label,t,n,m,n_out,dtype,shift", DECODE_TIE_CASES, ids=[c[0] for c in DECODE_TIE_CASES])
def test_decode_ties(kind, label, t, n, m, n_out, dtype, shift):
    dev = _dev()
    spec = wl.SPECS["decode"].with_(t=t, k=1024, n_out=n_out, n=n, m=m, dtype=dtype, score="magnitude",
                                    shift=shift, alpha=0.0, n_outliers=0)
    _, w = wl.make_inputs(spec)
    x = wl.adversarial_x(kind, t, spec.k, m, dtype, seed=t + n + m)
    pw = spa.prepare_weight(w.to(dev), 0.0)
    pr = oracle_for(spec, x, w)
    y, idx, nu = spa.sparse_linear_decode(x.to(dev), pw, _cfg(spec), want_idx=True)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), pr["idx"]), f"{label}/{kind}: decode masks differ"
    err = O.rowwise_error(f32(y), pr["y"])
    assert err <= O.TOLERANCE[dtype], (label, kind, err)


# The matrix-core path at a wide ragged output: a ragged last 64-row tile
# (3576 = 55 x 64 + 56), a ragged last 64-channel step and a last stage that
# overhangs k (1056 channels = 16.5 steps), one and two token blocks, with and
# without the shift and the variance factor.
MM16_CASES = [("t5_mag_mean", 5, "bf16", "magnitude", "token_mean", False, 2, 4),
              ("t16_clact_var", 16, "f16", "clact", "none", True, 16, 32),
              ("t17_weight", 17, "bf16", "weight", "none", False, 8, 16),
              ("t32_clact_var_mean", 32, "f16", "clact", "token_mean", True, 16, 32)]


@pytest.mark.parametrize("label,t,dtype,score,shift,var,n,m", MM16_CASES, ids=[c[0] for c in MM16_CASES])
def test_decode_matrix_core_wide_ragged(label, t, dtype, score, shift, var, n, m):
    dev = _dev()
    spec = wl.SPECS["batched"].with_(t=t, k=1056, n_out=3576, dtype=dtype, score=score, shift=shift,
                                     var_rescale=var, n=n, m=m, alpha=0.5 if score == "weight" else 0.0)
    x, w = wl.make_inputs(spec)
    pw = spa.prepare_weight(w.to(dev), spec.alpha, want_wt=False)
    f = f32(pw.chan_scale) if score == "weight" else None
    if f is not None:
        assert np.array_equal(f.view(np.uint32), O.channel_factor(f32(w), spec.alpha).view(np.uint32))
    pr = oracle_for(spec, x, w, f=f)
    y, idx, nu = spa.sparse_linear_decode(x.to(dev), pw, _cfg(spec), want_idx=True, want_nu=True)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), pr["idx"]), f"{label}: decode masks differ"
    assert np.allclose(f32(nu), pr["nu"], rtol=1e-6, atol=0), label
    err = O.rowwise_error(f32(y), pr["y"])
    assert err <= O.TOLERANCE[dtype], (label, err)


def test_decode_repeat_reuses_workspace():
    # Counters left at zero: a second call on the same workspace gives the same bytes.
    dev = _dev()
    spec = wl.SPECS["decode"].with_(t=1, k=2048, n_out=4096)
    x, w = wl.make_inputs(spec)
    pw = spa.prepare_weight(w.to(dev), spec.alpha)
    xd = x.to(dev)
    y1, _, _ = spa.sparse_linear_decode(xd, pw, _cfg(spec))
    y2, _, _ = spa.sparse_linear_decode(xd, pw, _cfg(spec))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_decode_workspaces_of_equal_size_do_not_mix():
    # two layouts that need the same number of workspace bytes (13056): the
    # binding keeps a workspace per layout, so neither call finds the other's
    # partial sums where its split counters should be zero
    dev = _dev()
    a = wl.SPECS["decode"].with_(t=1, k=1024, n_out=520, n=2, m=4, score="magnitude", shift="none", n_outliers=0)
    b = wl.SPECS["decode"].with_(t=2, k=256, n_out=136, n=2, m=4, score="magnitude", shift="none", n_outliers=0)
    sizes = {spa.workspace_bytes(1, s.t, s.k, s.n_out, torch.bfloat16, _cfg(s)) for s in (a, b)}
    assert len(sizes) == 1, sizes
    runs = []
    for s in (a, b):
        x, w = wl.make_inputs(s)
        runs.append((s, x.to(dev), spa.prepare_weight(w.to(dev), 0.0), oracle_for(s, x, w)))
    for _ in range(3):
        for s, xd, pw, pr in runs:
            y, idx, _ = spa.sparse_linear_decode(xd, pw, _cfg(s), want_idx=True)
            torch.cuda.synchronize()
            assert np.array_equal(idx.cpu().numpy(), pr["idx"])
            assert O.rowwise_error(f32(y), pr["y"]) <= O.TOLERANCE[s.dtype]


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
PREFILL_CASES = [s for s in wl.parity_specs() if s.dtype != "f32"]
for dt in ["bf16", "f16"]:
    for n, m in [(2, 4), (1, 4), (4, 8), (8, 16), (16, 32), (4, 4)]:
        PREFILL_CASES.append(wl.SPECS["prefill"].with_(name=f"pre_{dt}_{n}_{m}", t=77, k=320, n_out=300, dtype=dt,
                                                       n=n, m=m, n_outliers=3))
PREFILL_CASES.append(wl.SPECS["prefill"].with_(name="pre_weight_var", t=300, k=512, n_out=272, score="weight",
                                               alpha=0.5, var_rescale=True))
PREFILL_CASES.append(wl.SPECS["prefill"].with_(name="pre_given", t=40, k=256, n_out=520, shift="given"))
PREFILL_CASES.append(wl.SPECS["batched"].with_(name="pre_clact", t=96, k=512, n_out=264, n=2, m=4))
PREFILL_CASES.append(wl.SPECS["prefill"].with_(name="pre_one_row", t=1, k=128, n_out=8))
# squared ReLU applied by the library: CLACT with the token mean (the shift and
# column kernels), another n:m (dense matrix cores) and a long row
PREFILL_CASES.append(wl.SPECS["batched"].with_(name="pre_act_clact_mean", t=96, k=512, n_out=264, n=2, m=4,
                                               shift="token_mean", act="relu2", x_dist="normal"))
PREFILL_CASES.append(wl.SPECS["relu2_fused"].with_(name="pre_act_8_16", t=77, k=320, n_out=300, n=8, m=16))
PREFILL_CASES.append(wl.SPECS["relu2_fused"].with_(name="pre_act_long_row", t=40, k=8192, n_out=136,
                                                   shift="token_mean", var_rescale=True))
# more 256 x 256 tiles than one round of 256 CUs, the last round at most three
# quarters full: whole rounds of those tiles, then one round of 256 x 192
# tiles over the last columns (ragged token tile, ragged last column tile)
PREFILL_CASES.append(wl.SPECS["prefill"].with_(name="pre_tail_split", t=300, k=128, n_out=35000, n_outliers=2))
# k-step counts 1, 3 and 12 (the GEMMs run three k steps per loop turn with a
# peeled tail), and several ragged tiles in both directions
for n, m in [(2, 4), (4, 8)]:
    PREFILL_CASES.append(wl.SPECS["prefill"].with_(name=f"pre_k64_{n}_{m}", t=5, k=64, n_out=40, n=n, m=m))
    PREFILL_CASES.append(wl.SPECS["prefill"].with_(name=f"pre_k192_{n}_{m}", t=260, k=192, n_out=300, n=n, m=m))
    PREFILL_CASES.append(wl.SPECS["prefill"].with_(name=f"pre_tiles_{n}_{m}", t=600, k=768, n_out=1100, n=n, m=m,
                                                   n_outliers=8))


@pytest.mark.parametrize("spec", PREFILL_CASES, ids=[s.name for s in PREFILL_CASES])
def test_prefill_parity(spec):
    dev = _dev()
    x, w = wl.make_inputs(spec)
    eta_in = wl.make_eta(spec.t, 9) if spec.shift == "given" else None
    pw = spa.prepare_weight(w.to(dev), spec.alpha, want_wt=False)
    f = f32(pw.chan_scale) if spec.score == "weight" else None
    if f is not None:
        assert np.array_equal(f.view(np.uint32), O.channel_factor(f32(w), spec.alpha).view(np.uint32))
    pr = oracle_for(spec, x, w, f=f, eta_in=eta_in)
    cfg = _cfg(spec)
    ws = spa.workspace(2, spec.t, spec.k, spec.n_out, x.dtype, cfg, dev)
    y, idx, nu = spa.sparse_linear_prefill(x.to(dev), pw, cfg, eta_in=None if eta_in is None else eta_in.to(dev),
                                           want_idx=True, want_nu=True, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), pr["idx"]), "prefill masks differ"
    assert np.allclose(f32(nu), pr["nu"], rtol=1e-6, atol=0)
    # the operand the GEMM read, from the workspace: 2:4 packed values and
    # position words, or the masked rows of other n:m, bit for bit
    lay = spa.prefill_layout(spec.t, spec.k, x.dtype, cfg)
    if spec.n == 2 and spec.m == 4:
        vals, pos, _ = tiled_operand(ws, lay, spec.t, spec.k, False, spec.dtype)
        assert np.array_equal(vals, storage_bits(pr["vals"], spec.dtype)), "packed operand differs"
        assert np.array_equal(pos, pr["idx"]), "position words differ"
    else:
        raw = ws.cpu().numpy().view(np.uint8)[lay["vals"]:lay["vals"] + spec.t * spec.k * 2].view(np.uint16)
        masked = O.round_to_dtype(np.where(pr["keep"], pr["xhat"], np.float32(0.0)), spec.dtype)
        assert np.array_equal(raw.reshape(spec.t, spec.k), storage_bits(masked, spec.dtype)), "masked rows differ"
    err = O.rowwise_error(f32(y), pr["y"])
    assert err <= O.TOLERANCE[spec.dtype], err


def test_prefill_tail_split_eight_waves():
    # the same split behind the 8-wave tiles of rows over 8192 channels:
    # 1024 x 8256 -> 16640 is 260 tiles, 256 of them one round and the last
    # 256 columns two 192-wide tiles per token tile; sampled rows, every column
    dev = _dev()
    spec = wl.SPECS["prefill"].with_(name="pre_tail_split_8w", t=1024, k=8256, n_out=16640, n_outliers=4)
    x, w = wl.make_inputs(spec)
    pw = spa.prepare_weight(w.to(dev), spec.alpha, want_wt=False)
    y, idx, nu = spa.sparse_linear_prefill(x.to(dev), pw, _cfg(spec), want_idx=True, want_nu=True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 511, 700, 1022, 1023])
    pr = O.prune(f32(x[torch.as_tensor(rows)]), spec.dtype, spec.n, spec.m, score=spec.score, shift_mode=spec.shift)
    assert np.array_equal(idx.cpu().numpy()[rows], pr["idx"]), "positions differ on sampled rows"
    err = O.rowwise_error(f32(y)[rows], O.linear(pr, f32(w)))
    assert err <= O.TOLERANCE[spec.dtype], err


# A call that asks for neither positions nor nu, with no variance factor, as
# the benchmark makes it: 16-bit 2:4 rows of at most 16384 channels take the
# lean pruning pass (a persistent grid over the rows, a register ring).  The
# 2:4 cases above, plus rows of two, three and four 256-segment passes, a
# token count that gives each workgroup several rows, and the weight factor.
LEAN_CASES = [s for s in PREFILL_CASES if s.n == 2 and s.m == 4 and not s.var_rescale]
LEAN_CASES += [
    wl.SPECS["relu2"].with_(name="lean_k16384", t=24, k=16384, n_out=72),
    wl.SPECS["relu2_fused"].with_(name="lean_k12288_mean", t=19, k=12288, n_out=40, shift="token_mean"),
    wl.SPECS["prefill"].with_(name="lean_k8192_given", t=33, k=8192, n_out=48, shift="given"),
    wl.SPECS["prefill"].with_(name="lean_many_rows", t=3000, k=128, n_out=40),
    wl.SPECS["prefill"].with_(name="lean_weight", t=50, k=1024, n_out=96, score="weight", alpha=0.5),
]


@pytest.mark.parametrize("spec", LEAN_CASES, ids=[s.name for s in LEAN_CASES])
def test_prefill_operand_only(spec):
    dev = _dev()
    x, w = wl.make_inputs(spec)
    eta_in = wl.make_eta(spec.t, 9) if spec.shift == "given" else None
    print(f"[prefill operand only] {spec.name}: t={spec.t} k={spec.k} n_out={spec.n_out}", flush=True)
    pw = spa.prepare_weight(w.to(dev), spec.alpha, want_wt=False)
    f = f32(pw.chan_scale) if spec.score == "weight" else None
    pr = oracle_for(spec, x, w, f=f, eta_in=eta_in)
    cfg = _cfg(spec)
    ws = spa.workspace(2, spec.t, spec.k, spec.n_out, x.dtype, cfg, dev)
    y, idx, nu = spa.sparse_linear_prefill(x.to(dev), pw, cfg, eta_in=None if eta_in is None else eta_in.to(dev),
                                           ws=ws)
    torch.cuda.synchronize()
    assert idx is None and nu is None
    # every row: the packed values and position words, and the shift, bit for bit
    lay = spa.prefill_layout(spec.t, spec.k, x.dtype, cfg)
    vals, pos, _ = tiled_operand(ws, lay, spec.t, spec.k, False, spec.dtype)
    assert np.array_equal(pos, pr["idx"]), "position words differ"
    assert np.array_equal(vals, storage_bits(pr["vals"], spec.dtype)), "packed operand differs"
    eta = ws.cpu().numpy().view(np.uint8)[lay["eta"]:lay["eta"] + 4 * spec.t].view(np.float32)
    assert np.array_equal(eta.view(np.uint32), pr["eta"].view(np.uint32)), "shift differs"
    err = O.rowwise_error(f32(y), pr["y"])
    assert err <= O.TOLERANCE[spec.dtype], err

"""The decode entry point that allocates nothing (sparse_linear_decode_static).

It runs the same kernels as sparse_linear_decode on the library's static
per-GPU scratch.  Calls of decreasing size share that scratch; each must give
the workspace call's positions, nu and y bit for bit, and meet the oracle's
bar (positions bit for bit, y within the row-normwise tolerance).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import nm_oracle as O
from gpu_util import f32

pytestmark = pytest.mark.gpu

spa = pytest.importorskip("activation_sparsification_amd")

# one-token kernel (8 channel splits; then 16 with the variance sums), then
# the matrix-core path (20 tokens, then 3), then the fused kernel (float32):
# each call smaller than the one before, then the first again
CALLS = [
    ("decode_layer", wl.SPECS["decode"]),
    ("batched_t1", wl.SPECS["batched"].with_(t=1)),
    ("batched_t20", wl.SPECS["batched"].with_(t=20, k=2048, n_out=1000)),
    ("mm_t3", wl.SPECS["batched"].with_(t=3, k=1024, n_out=776)),
    ("fused_f32_t3", wl.SPECS["batched"].with_(t=3, k=512, n_out=136, dtype="f32")),
    ("decode_layer_again", wl.SPECS["decode"]),
]


def test_static_decode_matches_workspace_decode():
    assert torch.cuda.is_available(), "GPU tests need a device"
    dev = torch.device("cuda:0")
    for label, spec in CALLS:
        print(f"[no-alloc decode] {label}: t={spec.t} k={spec.k} n_out={spec.n_out} {spec.n}:{spec.m}", flush=True)
        x, w = wl.make_inputs(spec)
        xd = x.to(dev)
        pw = spa.prepare_weight(w.to(dev), spec.alpha, want_wt=spec.t <= 1 or spec.dtype == "f32")
        cfg = spa.PruneConfig(spec.n, spec.m, spec.score, spec.shift, spec.var_rescale, spec.act)
        y0, i0, n0 = spa.sparse_linear_decode(xd, pw, cfg, want_idx=True, want_nu=True)
        y1, i1, n1 = spa.sparse_linear_decode_static(xd, pw, cfg, want_idx=True, want_nu=True)
        torch.cuda.synchronize()
        assert torch.equal(i1, i0), label
        assert torch.equal(y1.view(torch.int16), y0.view(torch.int16)), label
        assert torch.equal(n1, n0), label
        f = O.channel_factor(f32(w), spec.alpha) if spec.score == "weight" else None
        pr = O.prune(f32(x), spec.dtype, spec.n, spec.m, score=spec.score, f=f, shift_mode=spec.shift,
                     var_rescale=spec.var_rescale)
        assert np.array_equal(i1.cpu().numpy(), pr["idx"]), label
        assert np.allclose(f32(n1), pr["nu"], rtol=1e-6, atol=0), label
        err = O.rowwise_error(f32(y1), O.linear(pr, f32(w)))
        assert err <= O.TOLERANCE[spec.dtype], (label, err)

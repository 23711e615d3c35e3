"""Seeded synthetic inputs for the N:M activation-pruned linear layer.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the pruning or linear-layer arithmetic, so both the CPU
oracle (through the tests) and the GPU path (through the tests and the
benchmark) can take their inputs from it without sharing any of the method.

Recipe, identical for every workload: one fresh
``numpy.random.Generator(PCG64(seed))``; draw the activation base values,
then the outlier channel indices (``rng.choice(K, n, replace=False)``, the
whole column multiplied over all tokens), then the weight, all in float64;
round to float32 (numpy, round-to-nearest-even) and then to the storage
dtype (torch ``.to``, round-to-nearest-even).

The five named workloads mirror the layer shapes of an 8B-class decoder
(hidden 4096, FFN 14336) on which the pages quote their results:

* ``tiny``     X[4,64] fp32 ~N(0,1), W[32,64] ~N(0,0.02); 2:4 magnitude.
* ``decode``   X[1,4096] bf16 = 0.5*t(df=3) with 8 outlier channels x20,
               W[14336,4096] ~N(0,0.02); 8:16, weight-aware alpha=0.5,
               per-token mean shift.
* ``prefill``  X[2048,4096] bf16 ~N(0,1) with 41 (1 %) outlier channels x10,
               W[14336,4096]; 2:4 magnitude, per-token mean shift.
* ``relu2``    X[4096,16384] bf16 = relu(z)^2, z ~N(-1,1) (about 84 % exact
               zeros), W[4096,16384]; 2:4 magnitude, no shift (the
               down-projection after a squared-ReLU FFN).
* ``batched``  X[T,14336] fp16 ~Laplace(0,0.3), T in {1,8,32},
               W[4096,14336]; 16:32, CLACT column score, variance rescale.
* ``relu2_fused``  the relu2 layer fed its pre-activation: X[4096,16384]
               bf16 = z ~N(-1,1) and the squared ReLU applied by the
               library (act "relu2") before it prunes and packs.
"""
from __future__ import annotations

import dataclasses
import itertools
import math
from typing import Optional

import numpy as np
import torch

_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shapes, distributions and pruning settings of one workload."""

    name: str
    t: int
    k: int
    n_out: int
    dtype: str            # "f32" | "f16" | "bf16"
    x_dist: str           # "normal" | "student_t3_half" | "relu2_shifted" | "preact_shifted" | "laplace"
    n_outliers: int
    outlier_gain: float
    n: int
    m: int
    score: str            # "magnitude" | "weight" | "clact"
    alpha: float
    shift: str            # "none" | "token_mean" | "given"
    var_rescale: bool
    w_std: float = 0.02
    act: str = "none"     # "none" | "relu2": x holds the pre-activation u

    def with_(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


SPECS = {
    "tiny": Spec("tiny", 4, 64, 32, "f32", "normal", 0, 1.0, 2, 4, "magnitude", 0.0, "none", False),
    "decode": Spec("decode", 1, 4096, 14336, "bf16", "student_t3_half", 8, 20.0, 8, 16, "weight", 0.5,
                   "token_mean", False),
    "prefill": Spec("prefill", 2048, 4096, 14336, "bf16", "normal", 41, 10.0, 2, 4, "magnitude", 0.0,
                    "token_mean", False),
    "relu2": Spec("relu2", 4096, 16384, 4096, "bf16", "relu2_shifted", 0, 1.0, 2, 4, "magnitude", 0.0,
                  "none", False),
    "batched": Spec("batched", 8, 14336, 4096, "f16", "laplace", 0, 1.0, 16, 32, "clact", 0.0, "none", True),
    "relu2_fused": Spec("relu2_fused", 4096, 16384, 4096, "bf16", "preact_shifted", 0, 1.0, 2, 4, "magnitude",
                        0.0, "none", False, act="relu2"),
}


def _draw_x(rng: np.random.Generator, spec: Spec) -> np.ndarray:
    shape = (spec.t, spec.k)
    if spec.x_dist == "normal":
        x = rng.standard_normal(shape)
    elif spec.x_dist == "student_t3_half":
        x = 0.5 * rng.standard_t(3.0, size=shape)
    elif spec.x_dist == "relu2_shifted":
        z = rng.normal(-1.0, 1.0, size=shape)
        x = np.square(np.maximum(z, 0.0))
    elif spec.x_dist == "laplace":
        x = rng.laplace(0.0, 0.3, size=shape)
    elif spec.x_dist == "preact_shifted":        # the up-projection output before max(0, .)^2
        x = rng.normal(-1.0, 1.0, size=shape)
    elif spec.x_dist == "relu2_standard":
        z = rng.standard_normal(shape)
        x = np.square(np.maximum(z, 0.0))
    else:
        raise ValueError(f"unknown activation distribution {spec.x_dist!r}")
    if spec.n_outliers:
        cols = rng.choice(spec.k, spec.n_outliers, replace=False)
        x[:, cols] *= spec.outlier_gain
    return x


def _to_storage(a64: np.ndarray, dtype: str) -> torch.Tensor:
    a32 = np.ascontiguousarray(a64.astype(np.float32))
    return torch.from_numpy(a32).to(_TORCH_DTYPES[dtype])


def make_inputs(spec: Spec, seed: int = 0, with_weight: bool = True):
    """Return ``(X, W)`` as CPU torch tensors in ``spec.dtype``.

    ``X`` is [t, k]; ``W`` is [n_out, k] (the layer computes ``y = x W^T``).
    ``W`` is None when ``with_weight`` is False (the draw order is kept, so X
    is the same either way).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _to_storage(_draw_x(rng, spec), spec.dtype)
    w = None
    if with_weight:
        w = _to_storage(rng.normal(0.0, spec.w_std, size=(spec.n_out, spec.k)), spec.dtype)
    return x, w


def make_eta(t: int, seed: int, scale: float = 0.1) -> torch.Tensor:
    """A given (static) per-token shift table, for the S-PTS hook."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    return torch.from_numpy(rng.normal(0.0, scale, size=(t,)).astype(np.float32))


def adversarial_x(kind: str, t: int, k: int, m: int, dtype: str, seed: int = 0) -> torch.Tensor:
    """Tie-heavy activation patterns for the top-N tie rule.

    kinds: ``equal`` (every block constant), ``zeros``, ``signed_pairs``
    (+v/-v alternating), ``signed_zero`` (+0/-0 mix), ``one_big`` (one large
    value, the rest tied), ``few_levels`` (values from a 3-level alphabet).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "equal":
        x = np.repeat(rng.standard_normal((t, k // m)), m, axis=1)
    elif kind == "zeros":
        x = np.zeros((t, k))
    elif kind == "signed_pairs":
        v = np.repeat(rng.standard_normal((t, k // 2)), 2, axis=1)
        x = v * np.tile([1.0, -1.0], k // 2)
    elif kind == "signed_zero":
        x = np.where(rng.random((t, k)) < 0.5, 0.0, -0.0)
        big = rng.random((t, k)) < 0.1
        x = np.where(big, rng.standard_normal((t, k)), x)
    elif kind == "one_big":
        x = np.full((t, k), 0.25)
        pos = rng.integers(0, m, size=(t, k // m))
        x = x.reshape(t, k // m, m)
        np.put_along_axis(x, pos[..., None], 4.0, axis=-1)
        x = x.reshape(t, k)
    elif kind == "few_levels":
        x = rng.choice(np.array([-1.0, 0.0, 0.5, 1.0]), size=(t, k))
    else:
        raise ValueError(kind)
    return _to_storage(x, dtype)


def random_positions(t: int, k: int, n: int, m: int, seed: int = 0) -> torch.Tensor:
    """Uniformly random kept positions: n distinct ascending in-block indices per m-block, uint8 [t, k*n/m]."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    if math.comb(m, n) <= 1 << 16:
        # one uniform draw per block from the list of every n-subset
        subsets = np.array(list(itertools.combinations(range(m), n)), dtype=np.uint8)
        pos = subsets[rng.integers(0, len(subsets), size=(t, k // m))]
    else:
        keys = rng.random((t, k // m, m))
        pos = np.sort(np.argsort(keys, axis=-1)[..., :n], axis=-1)
    return torch.from_numpy(np.ascontiguousarray(pos.reshape(t, k // m * n).astype(np.uint8)))


def parity_specs() -> list:
    """Reduced shapes that span several tiles of every kernel and end on a ragged tail."""
    return [
        SPECS["tiny"],
        SPECS["decode"].with_(name="decode_small", k=1024, n_out=1000),
        SPECS["prefill"].with_(name="prefill_small", t=200, k=512, n_out=520, n_outliers=5),
        SPECS["relu2"].with_(name="relu2_small", t=136, k=1024, n_out=264),
        SPECS["relu2_fused"].with_(name="relu2_fused_small", t=136, k=1024, n_out=264),
        SPECS["batched"].with_(name="batched_small_t1", t=1, k=1024, n_out=776),
        SPECS["batched"].with_(name="batched_small_t8", t=8, k=1024, n_out=776),
        SPECS["batched"].with_(name="batched_small_t32", t=32, k=1024, n_out=776),
    ]

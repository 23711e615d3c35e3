"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

from oracle import nm_oracle as O

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def storage_bits(v32: np.ndarray, dtype: str) -> np.ndarray:
    """Bit patterns of float32 values that are exactly representable in ``dtype``."""
    v32 = np.ascontiguousarray(v32, dtype=np.float32)
    if dtype == "f32":
        return v32.view(np.uint32)
    if dtype == "f16":
        return v32.astype(np.float16).view(np.uint16)
    return (v32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def tensor_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def check_ffn_masks(idx_gpu: np.ndarray, act_ref: np.ndarray, idx_ref: np.ndarray, rel_gap: float = 2.0 ** -5):
    """Masks of an activation the GPU forms from its own float32-accumulated
    up-projection.  Where the reference activation has a clear boundary in a
    block (2nd and 3rd largest more than rel_gap apart), the kept positions
    must match exactly; elsewhere the GPU's choice must be a top-2 of the
    reference up to that gap.  Returns the fraction of blocks that differ."""
    t, half = idx_gpu.shape
    nb = half // 2
    a = act_ref.reshape(t, nb, 4).astype(np.float64)
    g = idx_gpu.reshape(t, nb, 2).astype(np.int64)
    r = idx_ref.reshape(t, nb, 2).astype(np.int64)
    assert (g >= 0).all() and (g < 4).all() and (g[..., 0] < g[..., 1]).all(), "invalid positions"
    srt = -np.sort(-a, axis=-1)
    second, third = srt[..., 1], srt[..., 2]
    clear = second - third > rel_gap * np.maximum(second, 1e-30)
    differ = (g != r).any(axis=-1)
    assert not (differ & clear).any(), "mask differs where the boundary is clear"
    kept = np.take_along_axis(a, g, axis=-1).min(axis=-1)
    assert (kept >= third * (1 - rel_gap) - 1e-30).all(), "a kept value is below a dropped one"
    return float(differ.mean())


def oracle_for(spec, x_cpu, w_cpu, f=None, eta_in=None, rows=None):
    """Oracle prune (+ linear when w_cpu is given) for ``spec`` on CPU tensors."""
    x = f32(x_cpu) if rows is None else f32(x_cpu[rows])
    if spec.score == "weight" and f is None:
        f = O.channel_factor(f32(w_cpu), spec.alpha)
    eta = None if eta_in is None else (f32(eta_in) if rows is None else f32(eta_in[rows]))
    pr = O.prune(x, spec.dtype, spec.n, spec.m, score=spec.score, f=f, shift_mode=spec.shift, eta_in=eta,
                 var_rescale=spec.var_rescale, act=spec.act)
    if w_cpu is not None:
        pr["y"] = O.linear(pr, f32(w_cpu))
    pr["f"] = f
    return pr


def tiled_operand(ws: torch.Tensor, layout: dict, t: int, k: int, fp8: bool, dtype: str):
    """Read the 2:4 operand a prefill call left in its workspace (layout from
    ``spa.prefill_layout``): per token row, the kept entries in ascending channel
    order (e4m3 code bytes, or 16-bit storage bits), the kept in-block
    positions decoded from the nibble words, and the FP8 scales (or None)."""
    raw = ws.detach().cpu().numpy().view(np.uint8)
    steps, t_pad = k // 64, layout["t_pad"]
    if fp8:
        v = raw[layout["vals"]:layout["vals"] + steps * t_pad * 32].reshape(steps, t_pad, 32)
    else:
        v = raw[layout["vals"]:layout["vals"] + steps * t_pad * 64].view(np.uint16).reshape(steps, t_pad, 32)
    vals = v[:, :t, :].transpose(1, 0, 2).reshape(t, k // 2)
    words = raw[layout["meta"]:layout["meta"] + steps * t_pad * 8].view(np.uint16).reshape(steps, t_pad, 4)
    words = words[:, :t, :].transpose(1, 0, 2).reshape(t, k // 16).astype(np.int64)
    nib = (words[:, :, None] >> (4 * np.arange(4))[None, None, :]) & 0xF          # [t, k/16, 4 blocks]
    pos = np.stack([nib & 3, nib >> 2], axis=-1).reshape(t, k // 2).astype(np.uint8)
    scale = None
    if fp8:
        scale = raw[layout["scale"]:layout["scale"] + 4 * t].view(np.float32).copy()
    return vals, pos, scale

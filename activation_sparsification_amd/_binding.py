"""ctypes binding of ``libspa.so``: argument marshalling only.

Every step of the hot path runs in the library's HIP kernels.  torch is used
for device memory, dtypes and the current stream; nothing here computes.
If the library is missing, importing this module raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspa.so")

SPA_OK, SPA_ERR_INVALID, SPA_ERR_UNSUPPORTED, SPA_ERR_HIP, SPA_ERR_SCRATCH = 0, 1, 2, 3, 4
DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
SCORE = {"magnitude": 0, "weight": 1, "clact": 2}
SHIFT = {"none": 0, "token_mean": 1, "given": 2}
ACT = {"none": 0, "relu2": 1}
META = {"bitmap": 0, "comb": 1}
ENTRY_PRUNE, ENTRY_DECODE, ENTRY_PREFILL = 0, 1, 2


class SpaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lib().spa_status_str(status).decode()} (status {status})")
        self.status = status


class _Cfg(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("m", ctypes.c_int32), ("score", ctypes.c_int32),
                ("shift", ctypes.c_int32), ("var_rescale", ctypes.c_int32), ("act", ctypes.c_int32),
                ("var_state", ctypes.c_void_p), ("var_state_out", ctypes.c_void_p)]


class _PrefillLayout(ctypes.Structure):
    _fields_ = [("vals", ctypes.c_size_t), ("meta", ctypes.c_size_t), ("eta", ctypes.c_size_t),
                ("scale", ctypes.c_size_t), ("t_pad", ctypes.c_int32), ("bytes", ctypes.c_size_t)]


class _Weight(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("n_out", ctypes.c_int32), ("k", ctypes.c_int32),
                ("w", ctypes.c_void_p), ("wt", ctypes.c_void_p), ("chan_scale", ctypes.c_void_p),
                ("row_sum", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run `python -m activation_sparsification_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.spa_status_str.restype = ctypes.c_char_p
        L.spa_status_str.argtypes = [ctypes.c_int]
        L.spa_workspace_bytes.restype = sz
        L.spa_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(_Cfg)]
        L.spa_prefill_layout.restype = ctypes.c_int
        L.spa_prefill_layout.argtypes = [i32, i32, i32, ctypes.POINTER(_Cfg), ctypes.POINTER(_PrefillLayout)]
        L.prepare_weight.restype = ctypes.c_int
        L.prepare_weight.argtypes = [vp, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp]
        L.spa_eta_calibrate.restype = ctypes.c_int
        L.spa_eta_calibrate.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp, vp]
        L.spa_eta_table.restype = ctypes.c_int
        L.spa_eta_table.argtypes = [vp, vp, i32, vp, vp]
        L.spa_eta_lookup.restype = ctypes.c_int
        L.spa_eta_lookup.argtypes = [vp, i32, vp, i32, vp, vp]
        L.spa_ffn_workspace_bytes.restype = sz
        L.spa_ffn_workspace_bytes.argtypes = [i32, i32, i32]
        L.sparse_ffn_relu2_prefill.restype = ctypes.c_int
        L.sparse_ffn_relu2_prefill.argtypes = [vp, i32, ctypes.POINTER(_Weight), ctypes.POINTER(_Weight), vp, vp,
                                               vp, sz, vp]
        L.spa_amber_workspace_bytes.restype = sz
        L.spa_amber_workspace_bytes.argtypes = []
        L.prepare_amber.restype = ctypes.c_int
        L.prepare_amber.argtypes = [vp, i32, i32, i32, ctypes.c_float, vp, vp, sz, vp]
        L.prepare_weight_fp8.restype = ctypes.c_int
        L.prepare_weight_fp8.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.sparse_linear_prefill_fp8.restype = ctypes.c_int
        L.sparse_linear_prefill_fp8.argtypes = [vp, i32, ctypes.POINTER(_Weight), vp, vp, ctypes.POINTER(_Cfg), vp,
                                                vp, vp, vp, vp, sz, vp]
        L.spa_meta_row_bytes.restype = sz
        L.spa_meta_row_bytes.argtypes = [i32, i32, i32, i32]
        for name in ("spa_encode_meta", "spa_decode_meta"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp]
        L.prune_nm.restype = ctypes.c_int
        L.prune_nm.argtypes = [vp, i32, i32, i32, ctypes.POINTER(_Cfg), vp, vp, vp, vp, vp, vp, vp, sz, vp]
        for name in ("sparse_linear_decode", "sparse_linear_prefill"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [vp, i32, ctypes.POINTER(_Weight), ctypes.POINTER(_Cfg), vp, vp, vp, vp, vp, sz, vp]
        L.sparse_linear_decode_static.restype = ctypes.c_int
        L.sparse_linear_decode_static.argtypes = [vp, i32, ctypes.POINTER(_Weight), ctypes.POINTER(_Cfg), vp, vp,
                                                  vp, vp, vp]
        _lib = L
    return _lib


EXPORTS = ("prepare_weight", "prune_nm", "sparse_linear_decode", "sparse_linear_prefill",
           "spa_workspace_bytes", "spa_status_str", "spa_meta_row_bytes", "spa_encode_meta", "spa_decode_meta",
           "prepare_amber", "spa_amber_workspace_bytes", "spa_eta_calibrate", "spa_eta_table", "spa_eta_lookup",
           "sparse_ffn_relu2_prefill", "spa_ffn_workspace_bytes", "prepare_weight_fp8",
           "sparse_linear_prefill_fp8", "spa_prefill_layout", "sparse_linear_decode_static")


@dataclasses.dataclass(frozen=True)
class PruneConfig:
    """Keep ``n`` of every ``m`` channels; ``score`` / ``shift`` / ``act`` as in the C header."""
    n: int
    m: int
    score: str = "magnitude"
    shift: str = "none"
    var_rescale: int = 0          # 0, 1 (closed form) or 2 (running average: needs the two state tensors)
    act: str = "none"
    var_state: Optional[torch.Tensor] = None       # var_rescale == 2: float32 [t] state in
    var_state_out: Optional[torch.Tensor] = None   # var_rescale == 2: float32 [t] state out

    def c(self) -> _Cfg:
        return _Cfg(self.n, self.m, SCORE[self.score], SHIFT[self.shift], int(self.var_rescale), ACT[self.act],
                    _ptr(self.var_state), _ptr(self.var_state_out))


@dataclasses.dataclass
class PreparedWeight:
    w: torch.Tensor                      # [n_out, k]
    wt: Optional[torch.Tensor]           # [k, n_out]
    chan_scale: Optional[torch.Tensor]   # [k] float32
    row_sum: Optional[torch.Tensor]      # [n_out] float32

    @property
    def n_out(self) -> int:
        return self.w.shape[0]

    @property
    def k(self) -> int:
        return self.w.shape[1]

    def c(self, wt: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None) -> _Weight:
        wt = self.wt if wt is None else wt
        w = self.w if w is None else w
        return _Weight(DTYPE[self.w.dtype], self.n_out, self.k, _ptr(w), _ptr(wt), _ptr(self.chan_scale),
                       _ptr(self.row_sum))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, where: str):
    if status != SPA_OK:
        raise SpaError(status, where)


def _dev(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.device


def workspace_bytes(entry: int, t: int, k: int, n_out: int, dtype: torch.dtype, cfg: PruneConfig) -> int:
    c = cfg.c()
    return int(lib().spa_workspace_bytes(entry, t, k, n_out, DTYPE[dtype], ctypes.byref(c)))


def prefill_layout(t: int, k: int, dtype: torch.dtype, cfg: PruneConfig) -> dict:
    """Byte offsets of the pruned operand, positions, shift and FP8 scales in a prefill workspace."""
    c = cfg.c()
    out = _PrefillLayout()
    _check(lib().spa_prefill_layout(t, k, DTYPE[dtype], ctypes.byref(c), ctypes.byref(out)), "spa_prefill_layout")
    return {name: getattr(out, name) for name, _ in _PrefillLayout._fields_}


_WS_CACHE: dict = {}


def workspace(entry: int, t: int, k: int, n_out: int, dtype: torch.dtype, cfg: PruneConfig, device) -> Optional[torch.Tensor]:
    """A zero-filled workspace of the size the library asks for.

    Cached per device, entry point, sizes and the configuration fields that
    shape its layout: a decode workspace keeps split counters that a call
    leaves at zero for the next call of the same layout, but another layout
    of the same byte size could find its counters where partial sums were.
    """
    nbytes = workspace_bytes(entry, t, k, n_out, dtype, cfg)
    if nbytes == 0:
        return None
    key = (str(device), entry, nbytes, t, k, n_out, DTYPE[dtype], cfg.n, cfg.m, cfg.score, cfg.shift,
           int(cfg.var_rescale))
    ws = _WS_CACHE.get(key)
    if ws is None:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _WS_CACHE[key] = ws
    return ws


def prepare_weight(w: torch.Tensor, alpha: float = 0.0, want_wt: bool = True) -> PreparedWeight:
    """Channel-major copy, per-channel norm^alpha and row sums of W[n_out, k]."""
    dev = _dev(w)
    n_out, k = w.shape
    wt = torch.empty((k, n_out), dtype=w.dtype, device=dev) if want_wt else None
    cs = torch.empty(k, dtype=torch.float32, device=dev)
    rs = torch.empty(n_out, dtype=torch.float32, device=dev)
    _check(lib().prepare_weight(_ptr(w), DTYPE[w.dtype], n_out, k, float(alpha), _ptr(wt), _ptr(cs), _ptr(rs),
                                _stream(dev)), "prepare_weight")
    return PreparedWeight(w, wt, cs, rs)


def prune_nm(x: torch.Tensor, cfg: PruneConfig, chan_scale: Optional[torch.Tensor] = None,
             eta_in: Optional[torch.Tensor] = None, want_idx: bool = True):
    """Returns ``(vals [t, k*n/m], idx [t, k*n/m] uint8 or None, eta [t], nu [t])``."""
    dev = _dev(x)
    t, k = x.shape
    kept = k // cfg.m * cfg.n
    vals = torch.empty((t, kept), dtype=x.dtype, device=dev)
    idx = torch.empty((t, kept), dtype=torch.uint8, device=dev) if want_idx else None
    eta = torch.empty(t, dtype=torch.float32, device=dev)
    nu = torch.empty(t, dtype=torch.float32, device=dev)
    ws = workspace(ENTRY_PRUNE, t, k, 0, x.dtype, cfg, dev)
    c = cfg.c()
    _check(lib().prune_nm(_ptr(x), DTYPE[x.dtype], t, k, ctypes.byref(c), _ptr(chan_scale), _ptr(eta_in),
                          _ptr(vals), _ptr(idx), _ptr(eta), _ptr(nu), _ptr(ws), 0 if ws is None else ws.numel(),
                          _stream(dev)), "prune_nm")
    return vals, idx, eta, nu


def sparse_ffn_relu2_prefill(x: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor, want_idx: bool = False,
                             out: Optional[torch.Tensor] = None):
    """y = prune24(max(x W_up^T, 0)^2) W_down^T; returns (y [t, n_out], idx [t, ffn/2] uint8 or None)."""
    dev = _dev(x)
    t, hidden = x.shape
    ffn = w_up.shape[0]
    n_out = w_down.shape[0]
    y = torch.empty((t, n_out), dtype=x.dtype, device=dev) if out is None else out
    idx = torch.empty((t, ffn // 2), dtype=torch.uint8, device=dev) if want_idx else None
    nb = int(lib().spa_ffn_workspace_bytes(t, ffn, DTYPE[x.dtype]))
    key = (str(dev), "ffn", nb)
    ws = _WS_CACHE.get(key)
    if ws is None:
        ws = torch.zeros(max(nb, 1), dtype=torch.uint8, device=dev)
        _WS_CACHE[key] = ws
    up = _Weight(DTYPE[w_up.dtype], ffn, hidden, _ptr(w_up), None, None, None)
    dn = _Weight(DTYPE[w_down.dtype], n_out, ffn, _ptr(w_down), None, None, None)
    _check(lib().sparse_ffn_relu2_prefill(_ptr(x), t, ctypes.byref(up), ctypes.byref(dn), _ptr(y), _ptr(idx), _ptr(ws),
                                          nb, _stream(dev)), "sparse_ffn_relu2_prefill")
    return y, idx


class EtaCalibration:
    """Static shift table (S-PTS): add calibration batches, then read the table."""

    def __init__(self, vocab: int, device):
        self.vocab = vocab
        self.sums = torch.zeros(vocab, dtype=torch.float64, device=device)
        self.counts = torch.zeros(vocab, dtype=torch.int32, device=device)

    def add(self, x: torch.Tensor, token_ids: torch.Tensor) -> None:
        dev = _dev(x)
        t, k = x.shape
        ids = token_ids.to(device=dev, dtype=torch.int32).contiguous()
        _check(lib().spa_eta_calibrate(_ptr(x), DTYPE[x.dtype], t, k, _ptr(ids), self.vocab, _ptr(self.sums),
                                       _ptr(self.counts), _stream(dev)), "spa_eta_calibrate")

    def table(self) -> torch.Tensor:
        dev = self.sums.device
        out = torch.empty(self.vocab, dtype=torch.float32, device=dev)
        _check(lib().spa_eta_table(_ptr(self.sums), _ptr(self.counts), self.vocab, _ptr(out), _stream(dev)),
               "spa_eta_table")
        return out


def eta_lookup(table: torch.Tensor, token_ids: torch.Tensor) -> torch.Tensor:
    """Per-token static shift: the table entry of each token id (0 outside the table)."""
    dev = _dev(table)
    ids = token_ids.to(device=dev, dtype=torch.int32).contiguous()
    out = torch.empty(ids.numel(), dtype=torch.float32, device=dev)
    _check(lib().spa_eta_lookup(_ptr(table), table.numel(), _ptr(ids), ids.numel(), _ptr(out), _stream(dev)),
           "spa_eta_lookup")
    return out


def prepare_amber(w: torch.Tensor, alpha: float = 1.0) -> torch.Tensor:
    """Amber-Pruner channel factor of W[n_out, k]: a float32 [k] chan_scale for the weight-aware score."""
    dev = _dev(w)
    n_out, k = w.shape
    out = torch.empty(k, dtype=torch.float32, device=dev)
    nb = int(lib().spa_amber_workspace_bytes())
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    _check(lib().prepare_amber(_ptr(w), DTYPE[w.dtype], n_out, k, float(alpha), _ptr(out), _ptr(ws), nb,
                               _stream(dev)), "prepare_amber")
    return out


def meta_row_bytes(k: int, n: int, m: int, fmt: str = "comb") -> int:
    """Bytes of packed block codes per token row (0 for invalid arguments)."""
    return int(lib().spa_meta_row_bytes(k, n, m, META[fmt]))


def encode_meta(idx: torch.Tensor, n: int, m: int, fmt: str = "comb") -> torch.Tensor:
    """uint8 in-block positions [t, k*n/m] -> packed codes, uint32 [t, row_bytes/4] (as int32 storage)."""
    dev = _dev(idx)
    t, kept = idx.shape
    k = kept // n * m
    words = meta_row_bytes(k, n, m, fmt) // 4
    codes = torch.zeros((t, words), dtype=torch.int32, device=dev)
    _check(lib().spa_encode_meta(_ptr(idx), t, k, n, m, META[fmt], _ptr(codes) if codes.numel() else None,
                                 _stream(dev)), "spa_encode_meta")
    return codes


def decode_meta(codes: torch.Tensor, k: int, n: int, m: int, fmt: str = "comb") -> torch.Tensor:
    """Packed codes [t, row_words] -> uint8 in-block positions [t, k*n/m]."""
    dev = _dev(codes)
    t = codes.shape[0]
    idx = torch.empty((t, k // m * n), dtype=torch.uint8, device=dev)
    _check(lib().spa_decode_meta(_ptr(codes) if codes.numel() else None, t, k, n, m, META[fmt], _ptr(idx),
                                 _stream(dev)), "spa_decode_meta")
    return idx


def _linear(fn_name: str, entry: int, x: torch.Tensor, pw: PreparedWeight, cfg: PruneConfig,
            eta_in: Optional[torch.Tensor], want_idx: bool, want_nu: bool, out: Optional[torch.Tensor],
            ws: Optional[torch.Tensor], wt: Optional[torch.Tensor] = None):
    dev = _dev(x)
    t, k = x.shape
    y = torch.empty((t, pw.n_out), dtype=x.dtype, device=dev) if out is None else out
    idx = torch.empty((t, k // cfg.m * cfg.n), dtype=torch.uint8, device=dev) if want_idx else None
    nu = torch.empty(t, dtype=torch.float32, device=dev) if want_nu else None
    if ws is None:
        ws = workspace(entry, t, k, pw.n_out, x.dtype, cfg, dev)
    c = cfg.c()
    wd = pw.c(wt=wt)
    st = getattr(lib(), fn_name)(_ptr(x), t, ctypes.byref(wd), ctypes.byref(c), _ptr(eta_in), _ptr(y), _ptr(idx),
                                 _ptr(nu), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
    _check(st, fn_name)
    return y, idx, nu


def sparse_linear_decode(x, pw: PreparedWeight, cfg: PruneConfig, eta_in=None, want_idx=False, want_nu=False,
                         out=None, ws=None, wt=None):
    """Fused prune + row-skipping GEMV for 1..32 tokens.  Returns ``(y, idx, nu)``."""
    return _linear("sparse_linear_decode", ENTRY_DECODE, x, pw, cfg, eta_in, want_idx, want_nu, out, ws, wt)


def sparse_linear_decode_static(x, pw: PreparedWeight, cfg: PruneConfig, eta_in=None, want_idx=False, want_nu=False,
                                out=None, wt=None):
    """sparse_linear_decode on the library's static per-GPU scratch (no workspace).  Returns ``(y, idx, nu)``."""
    dev = _dev(x)
    t, k = x.shape
    y = torch.empty((t, pw.n_out), dtype=x.dtype, device=dev) if out is None else out
    idx = torch.empty((t, k // cfg.m * cfg.n), dtype=torch.uint8, device=dev) if want_idx else None
    nu = torch.empty(t, dtype=torch.float32, device=dev) if want_nu else None
    c = cfg.c()
    wd = pw.c(wt=wt)
    _check(lib().sparse_linear_decode_static(_ptr(x), t, ctypes.byref(wd), ctypes.byref(c), _ptr(eta_in), _ptr(y),
                                             _ptr(idx), _ptr(nu), _stream(dev)), "sparse_linear_decode_static")
    return y, idx, nu


def sparse_linear_prefill(x, pw: PreparedWeight, cfg: PruneConfig, eta_in=None, want_idx=False, want_nu=False,
                          out=None, ws=None):
    """Prune/pack pass + matrix-core GEMM (sparse MFMA for 2:4).  Returns ``(y, idx, nu)``."""
    return _linear("sparse_linear_prefill", ENTRY_PREFILL, x, pw, cfg, eta_in, want_idx, want_nu, out, ws)


@dataclasses.dataclass
class Fp8Weight:
    """e4m3 codes of a weight, one float32 scale per output row (prepare_weight_fp8)."""
    codes: torch.Tensor                  # [n_out, k] uint8
    scale: torch.Tensor                  # [n_out] float32


def prepare_weight_fp8(w: torch.Tensor) -> Fp8Weight:
    """Row-scaled e4m3 copy of a 16-bit weight ``[n_out, k]`` for the FP8 2:4 prefill."""
    dev = _dev(w)
    n_out, k = w.shape
    codes = torch.empty((n_out, k), dtype=torch.uint8, device=dev)
    scale = torch.empty(n_out, dtype=torch.float32, device=dev)
    _check(lib().prepare_weight_fp8(_ptr(w), DTYPE[w.dtype], n_out, k, _ptr(codes), _ptr(scale), _stream(dev)),
           "prepare_weight_fp8")
    return Fp8Weight(codes, scale)


def sparse_linear_prefill_fp8(x, pw: PreparedWeight, w8: Fp8Weight, cfg: PruneConfig, eta_in=None, want_idx=False,
                              want_nu=False, out=None, ws=None):
    """2:4 prefill with FP8 operands (pruning pass + FP8 sparse MFMA GEMM).  Returns ``(y, idx, nu)``."""
    dev = _dev(x)
    t, k = x.shape
    y = torch.empty((t, pw.n_out), dtype=x.dtype, device=dev) if out is None else out
    idx = torch.empty((t, k // cfg.m * cfg.n), dtype=torch.uint8, device=dev) if want_idx else None
    nu = torch.empty(t, dtype=torch.float32, device=dev) if want_nu else None
    if ws is None:
        ws = workspace(ENTRY_PREFILL, t, k, pw.n_out, x.dtype, cfg, dev)
    c = cfg.c()
    wd = pw.c()
    st = lib().sparse_linear_prefill_fp8(_ptr(x), t, ctypes.byref(wd), _ptr(w8.codes), _ptr(w8.scale),
                                         ctypes.byref(c), _ptr(eta_in), _ptr(y), _ptr(idx), _ptr(nu), _ptr(ws),
                                         0 if ws is None else ws.numel(), _stream(dev))
    _check(st, "sparse_linear_prefill_fp8")
    return y, idx, nu


class PreparedCall:
    """A library call with every argument marshalled once (for tight loops and timing).

    ``__call__`` issues exactly one C call on the stream that was current at
    construction; outputs land in the tensors given here.
    """

    def __init__(self, fn_name: str, x, pw: PreparedWeight, cfg: PruneConfig, y, ws, eta_in=None, idx=None,
                 nu=None, wt=None, w=None, w8: Optional["Fp8Weight"] = None):
        self._keep = (x, pw, y, ws, eta_in, idx, nu, wt, w, w8)
        self._cfg = cfg.c()
        self._wd = pw.c(wt=wt, w=w)
        self._fn = getattr(lib(), fn_name)
        self._name = fn_name
        t = x.shape[0]
        fp8 = fn_name == "sparse_linear_prefill_fp8"
        if fp8 != (w8 is not None):
            raise ValueError("the FP8 prefill takes the weight's FP8 codes (w8), the other calls do not")
        head = (_ptr(x), t, ctypes.byref(self._wd))
        if fp8:
            head += (_ptr(w8.codes), _ptr(w8.scale))
        self._args = head + (ctypes.byref(self._cfg), _ptr(eta_in), _ptr(y), _ptr(idx), _ptr(nu), _ptr(ws),
                             0 if ws is None else ws.numel(), _stream(x.device))

    def __call__(self):
        st = self._fn(*self._args)
        if st != SPA_OK:
            raise SpaError(st, self._name)

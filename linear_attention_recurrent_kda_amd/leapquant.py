"""Python binding of the LeapQuant C ABI (include/leapquant.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libleapquant.so. PyTorch supplies device memory and the stream;
each call is enqueued on torch's current stream. Importing this module fails
loudly when the HIP library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libleapquant.so")

LQ_OK = 0
LQ_ERR_NULL, LQ_ERR_SHAPE, LQ_ERR_BITS, LQ_ERR_CONFIG, LQ_ERR_LAUNCH, LQ_ERR_ALIGN = -1, -2, -3, -4, -5, -6
LQ_ACT_F32, LQ_ACT_BF16 = 0, 1
LQ_DEVERR_BUFFER_FULL, LQ_DEVERR_BAD_SEQ, LQ_DEVERR_BAD_LEN = 1, 2, 4
LQ_STATE_NBUF = 8
STATE_FIELDS = ("codes", "row_scale", "col_scale", "ent_k", "ent_u", "ent_g", "buf_len", "err")

EXPORTS = ("lq_state_sizes", "leapquant_encode", "leapquant_decode_step", "leapquant_decode_step_at",
           "leapquant_decode_close_at", "leapquant_window_close",
           "gdn_decode_fp32_baseline", "leapquant_prefill", "lq_snapshot_bytes", "leapquant_snapshot",
           "leapquant_restore", "leapquant_dequantize", "lq_close_list", "lq_status_string")


class CDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "heads", "d_k", "d_v", "w_max", "n_comp", "bits", "decay_per_channel", "act_dtype",
        "smoothing", "power_iters", "warm_start")]


class CState(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in STATE_FIELDS]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"LeapQuant HIP library not built: {path} is missing "
                          "(run python -m linear_attention_recurrent_kda_amd.build)")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pd, ps = ctypes.POINTER(CDims), ctypes.POINTER(CState)
    sig = {
        "lq_state_sizes": (ctypes.c_int, [pd, ctypes.POINTER(SZ)]),
        "leapquant_encode": (ctypes.c_int, [pd, P, ps, P, P]),
        "leapquant_decode_step": (ctypes.c_int, [pd, ps, P, P, P, P, P, P, P]),
        "leapquant_decode_step_at": (ctypes.c_int, [pd, ps, I32, P, P, P, P, P, P, P]),
        "leapquant_decode_close_at": (ctypes.c_int, [pd, ps, I32, P, P, P, P, P, P, P, P]),
        "leapquant_window_close": (ctypes.c_int, [pd, ps, P, I32, P, P]),
        "gdn_decode_fp32_baseline": (ctypes.c_int, [pd, P, P, P, P, P, P, P, P]),
        "leapquant_prefill": (ctypes.c_int, [pd, P, I32, P, P, P, P, P, P, ps, P]),
        "lq_snapshot_bytes": (ctypes.c_int, [pd, ctypes.POINTER(SZ)]),
        "leapquant_snapshot": (ctypes.c_int, [pd, ps, P, I32, P, P]),
        "leapquant_restore": (ctypes.c_int, [pd, ps, P, I32, P, P]),
        "leapquant_dequantize": (ctypes.c_int, [pd, ps, P, P]),
        "lq_close_list": (I32, [P, P, I32, I64, P]),
        "lq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = load_library()


class LeapQuantError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def status_string(status: int) -> str:
    return _lib.lq_status_string(int(status)).decode()


def _check(fn: str, rc: int) -> None:
    if rc != LQ_OK:
        raise LeapQuantError(fn, rc)


@dataclass(frozen=True)
class Dims:
    """Problem shape and method parameters (mirrors lq_dims)."""

    batch: int
    heads: int
    d: int
    w_max: int = 16
    n_comp: int = 4
    bits: int = 8
    kda: bool = False
    bf16: bool = False
    smoothing: bool = True
    power_iters: int = 4
    warm_start: bool = False

    def c(self) -> CDims:
        return CDims(self.batch, self.heads, self.d, self.d, self.w_max, self.n_comp, self.bits,
                     int(self.kda), LQ_ACT_BF16 if self.bf16 else LQ_ACT_F32, int(self.smoothing),
                     self.power_iters, int(self.warm_start))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() or None


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def state_sizes(dims: Dims) -> Dict[str, int]:
    out = (ctypes.c_size_t * LQ_STATE_NBUF)()
    cd = dims.c()
    _check("lq_state_sizes", _lib.lq_state_sizes(ctypes.byref(cd), out))
    return dict(zip(STATE_FIELDS, (int(x) for x in out)))


def close_list(win_len, win_off, step: int):
    """Host schedule: sequences whose window ends with token `step`."""
    import numpy as np
    wl = np.ascontiguousarray(win_len, np.int32)
    wo = np.ascontiguousarray(win_off, np.int32)
    out = np.empty(max(len(wl), 1), np.int32)
    n = _lib.lq_close_list(wl.ctypes.data, wo.ctypes.data, len(wl), int(step), out.ctypes.data)
    if n < 0:
        raise LeapQuantError("lq_close_list", n)
    return out[:n].copy()


class State:
    """Device buffers of a LeapQuant state (all heads), allocated with torch."""

    def __init__(self, dims: Dims, device="cuda"):
        self.dims = dims
        sz = state_sizes(dims)
        BH, D, W, r = dims.batch * dims.heads, dims.d, dims.w_max, dims.n_comp
        f32 = dict(dtype=torch.float32, device=device)
        self.codes = torch.zeros((BH, D, D * dims.bits // 8), dtype=torch.int8, device=device)
        self.row_scale = torch.ones((BH, D), **f32)
        self.col_scale = torch.zeros((BH, D), **f32)
        # entries 0..r-1: compensators; r..r+W-1: buffered tokens (with bf16
        # activations a token's key row holds its bf16 key in the row's first
        # d * 2 bytes; compensator rows are fp32)
        self.ent_k = torch.zeros((BH, r + W, D), **f32)
        self.ent_u = torch.zeros((BH, r + W, D), **f32)
        self.ent_g = torch.zeros((BH, r + W, D) if dims.kda else (BH, r + W), **f32)
        self.buf_len = torch.zeros((BH,), dtype=torch.int32, device=device)
        self.err = torch.zeros((1,), dtype=torch.int32, device=device)
        for name in STATE_FIELDS:
            t = getattr(self, name)
            assert t.numel() * t.element_size() == sz[name], (name, t.shape, sz[name])

    def c(self) -> CState:
        return CState(*[_ptr(getattr(self, n)) for n in STATE_FIELDS])

    # views of the entry arrays
    @property
    def comp_k(self) -> torch.Tensor:
        return self.ent_k[:, :self.dims.n_comp]

    @property
    def comp_u(self) -> torch.Tensor:
        return self.ent_u[:, :self.dims.n_comp]

    @property
    def buf_k(self) -> torch.Tensor:
        """The buffered tokens' key rows as stored (bf16 activations: bf16 keys
        in each row's first half)."""
        return self.ent_k[:, self.dims.n_comp:]

    @property
    def buf_u(self) -> torch.Tensor:
        return self.ent_u[:, self.dims.n_comp:]

    @property
    def buf_g(self) -> torch.Tensor:
        return self.ent_g[:, self.dims.n_comp:]

    def nbytes(self) -> int:
        return sum(getattr(self, n).numel() * getattr(self, n).element_size() for n in STATE_FIELDS)


def encode(dims: Dims, S: torch.Tensor, st: State, dbg_residual: Optional[torch.Tensor] = None) -> None:
    """S: fp32 [B*H][d_v][d_k] (transposed dense states)."""
    cd, cs = dims.c(), st.c()
    _check("leapquant_encode", _lib.leapquant_encode(ctypes.byref(cd), _ptr(S), ctypes.byref(cs),
                                                     _ptr(dbg_residual), _stream()))


def decode_step(dims: Dims, st: State, q, k, v, g, beta, o) -> None:
    cd, cs = dims.c(), st.c()
    _check("leapquant_decode_step", _lib.leapquant_decode_step(
        ctypes.byref(cd), ctypes.byref(cs), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o),
        _stream()))


def decode_step_at(dims: Dims, st: State, n: int, q, k, v, g, beta, o) -> None:
    """decode_step for a state whose every head holds n buffered tokens."""
    cd, cs = dims.c(), st.c()
    _check("leapquant_decode_step_at", _lib.leapquant_decode_step_at(
        ctypes.byref(cd), ctypes.byref(cs), int(n), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(o), _stream()))


def decode_close_at(dims: Dims, st: State, n: int, q, k, v, g, beta, o,
                    dbg_residual: Optional[torch.Tensor] = None) -> None:
    """The window's last token (every head holding n buffered tokens) and the
    close of every sequence, in one launch."""
    cd, cs = dims.c(), st.c()
    _check("leapquant_decode_close_at", _lib.leapquant_decode_close_at(
        ctypes.byref(cd), ctypes.byref(cs), int(n), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(o), _ptr(dbg_residual), _stream()))


def window_close(dims: Dims, st: State, seq_ids: Optional[torch.Tensor] = None, n_seq: int = 0,
                 dbg_residual: Optional[torch.Tensor] = None) -> None:
    """seq_ids: device int32 tensor of sequence ids, or None for every sequence."""
    cd, cs = dims.c(), st.c()
    if seq_ids is not None and n_seq == 0:
        n_seq = seq_ids.numel()
    _check("leapquant_window_close", _lib.leapquant_window_close(
        ctypes.byref(cd), ctypes.byref(cs), _ptr(seq_ids), int(n_seq), _ptr(dbg_residual), _stream()))


def fp32_baseline_step(dims: Dims, S: torch.Tensor, q, k, v, g, beta, o) -> None:
    cd = dims.c()
    _check("gdn_decode_fp32_baseline", _lib.gdn_decode_fp32_baseline(
        ctypes.byref(cd), _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o), _stream()))


def prefill(dims: Dims, S: torch.Tensor, q, k, v, g, beta, o, st: Optional[State] = None) -> None:
    """Exact recurrence over a time-major prompt chunk (q, k, v: [L][B*H][d]; g:
    [L][B*H] or [L][B*H][d]; beta: [L][B*H]; o: [L][B*H][d]) on the fp32 state S
    ([B*H][d_v][d_k], in/out); then encode S into st when st is given."""
    cd = dims.c()
    n_tokens = 0 if q is None else int(q.shape[0])
    cs = st.c() if st is not None else None
    _check("leapquant_prefill", _lib.leapquant_prefill(
        ctypes.byref(cd), _ptr(S), n_tokens, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o),
        ctypes.byref(cs) if cs is not None else None, _stream()))


def snapshot_bytes(dims: Dims) -> int:
    """Bytes of one head's snapshot record."""
    out = ctypes.c_size_t()
    cd = dims.c()
    _check("lq_snapshot_bytes", _lib.lq_snapshot_bytes(ctypes.byref(cd), ctypes.byref(out)))
    return int(out.value)


def snapshot(dims: Dims, st: State, snap: torch.Tensor, seq_ids: Optional[torch.Tensor] = None) -> None:
    """Copy the listed sequences' window-boundary state into snap ([n][H][record] bytes)."""
    cd, cs = dims.c(), st.c()
    n = 0 if seq_ids is None else seq_ids.numel()
    _check("leapquant_snapshot", _lib.leapquant_snapshot(ctypes.byref(cd), ctypes.byref(cs), _ptr(seq_ids), n,
                                                         _ptr(snap), _stream()))


def restore(dims: Dims, st: State, snap: torch.Tensor, seq_ids: Optional[torch.Tensor] = None) -> None:
    cd, cs = dims.c(), st.c()
    n = 0 if seq_ids is None else seq_ids.numel()
    _check("leapquant_restore", _lib.leapquant_restore(ctypes.byref(cd), ctypes.byref(cs), _ptr(seq_ids), n,
                                                       _ptr(snap), _stream()))


def dequantize(dims: Dims, st: State, out: torch.Tensor) -> None:
    cd, cs = dims.c(), st.c()
    _check("leapquant_dequantize", _lib.leapquant_dequantize(ctypes.byref(cd), ctypes.byref(cs),
                                                             _ptr(out), _stream()))


def raw_call(name: str, *args) -> int:
    """Call an exported entry point with ctypes arguments; returns its status (tests)."""
    return getattr(_lib, name)(*args)

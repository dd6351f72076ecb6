"""Host-side decode loop over the C ABI: window schedule, close lists, uploads.

A Decoder owns one LeapQuant state (all B*H heads) and advances it one token
at a time: decode_step for every head, then window_close for the sequences
whose window ends with that token. Window ends are known on the host in
advance ((offset + t + 1) % W == 0 per sequence), so the close lists for one
schedule period are computed once and kept on the device; no step needs a
device-to-host read.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch

from . import leapquant as lqk
from .workloads import Workload, window_lengths, window_offsets


def dims_for(wl: Workload, bits: Optional[int] = None) -> lqk.Dims:
    return lqk.Dims(batch=wl.batch, heads=wl.heads, d=wl.d_k, w_max=wl.w_max, n_comp=wl.n_comp,
                    bits=wl.bits if bits is None else bits, kda=wl.kda, bf16=wl.act_bf16,
                    smoothing=wl.smoothing, power_iters=wl.power_iters, warm_start=wl.warm_start)


def upload_tokens(tok: Dict[str, np.ndarray], bf16: bool, device="cuda") -> Dict[str, torch.Tensor]:
    """Token inputs [n][S][H][...] from the workload stream -> contiguous device tensors with a
    leading step axis (the kernels read [B][H][d] per step)."""
    out = {}
    for name in ("q", "k", "v"):
        if bf16:
            arr = np.ascontiguousarray(tok[name + "16"]).view(np.int16)
            out[name] = torch.from_numpy(arr).to(device).view(torch.bfloat16)
        else:
            out[name] = torch.from_numpy(np.ascontiguousarray(tok[name])).to(device)
    out["g"] = torch.from_numpy(np.ascontiguousarray(tok["g"])).to(device)
    out["beta"] = torch.from_numpy(np.ascontiguousarray(tok["beta"])).to(device)
    return out


def states_to_device(S_math: np.ndarray, device="cuda") -> torch.Tensor:
    """Math-layout fp32 states [..][d_k][d_v] -> device [B*H][d_v][d_k] (transposed)."""
    d_k, d_v = S_math.shape[-2:]
    S = np.ascontiguousarray(np.swapaxes(S_math.reshape(-1, d_k, d_v), 1, 2), dtype=np.float32)
    return torch.from_numpy(S).to(device)


def buffered_tokens(win_len: np.ndarray, win_off: np.ndarray, t: int) -> np.ndarray:
    """Per sequence, the tokens its buffer holds before token t (counted from
    the encode). A sequence starts at offset o inside its first window with an
    empty buffer, so before its first close it holds t tokens and afterwards
    (t + o) mod W."""
    win_len, win_off = np.asarray(win_len, np.int64), np.asarray(win_off, np.int64)
    return np.where(t + win_off < win_len, t, (t + win_off) % win_len)


class Decoder:
    """The decode schedule of one state set: window lengths and offsets per
    sequence, the close lists they imply, and a token counter. With fuse, a
    token after which every sequence closes, all at the same window position,
    is taken inside the close (leapquant_decode_close_at) by step()."""

    def __init__(self, dims: lqk.Dims, win_len: np.ndarray, win_off: np.ndarray, device="cuda",
                 fuse: bool = True):
        self.dims = dims
        self.fuse = fuse
        self.state = lqk.State(dims, device)
        self.win_len = np.asarray(win_len, np.int32)
        self.win_off = np.asarray(win_off, np.int32)
        assert len(self.win_len) == dims.batch and np.all(self.win_len <= dims.w_max)
        self.period = int(np.lcm.reduce(self.win_len)) if dims.batch else 1
        lists = [lqk.close_list(self.win_len, self.win_off, t) for t in range(self.period)]
        self._close_n = [len(x) for x in lists]
        self._close_at = np.cumsum([0] + self._close_n[:-1]).tolist()
        flat = np.concatenate(lists + [np.zeros(1, np.int32)]).astype(np.int32)
        self._close_ids = torch.from_numpy(flat).to(device)
        self._all = all(n == dims.batch for n in self._close_n if n)
        self.t = 0
        self.o = torch.empty((dims.batch * dims.heads, dims.d), dtype=torch.float32, device=device)

    def encode(self, S_dev: torch.Tensor, dbg: Optional[torch.Tensor] = None) -> None:
        lqk.encode(self.dims, S_dev, self.state, dbg)
        self.t = 0

    def closes_at(self, t: int) -> int:
        return self._close_n[t % self.period]

    def position(self, t: int) -> int:
        """Tokens every sequence's buffer holds before token t, when all hold
        the same number, else -1."""
        n = buffered_tokens(self.win_len, self.win_off, t)
        return int(n[0]) if len(n) and np.all(n == n[0]) else -1

    def fused_at(self, t: int) -> int:
        """The window position of token t when every sequence closes after it,
        all at one position (so one launch can take the token and the close),
        else -1."""
        if not self.fuse or self.closes_at(t) != self.dims.batch:
            return -1
        return self.position(t)

    def decode(self, t: int, q, k, v, g, beta, o) -> None:
        """The decode step of token t: with the position given to the kernel
        when every sequence is at the same one."""
        n = self.position(t)
        if n >= 0:
            lqk.decode_step_at(self.dims, self.state, n, q, k, v, g, beta, o)
        else:
            lqk.decode_step(self.dims, self.state, q, k, v, g, beta, o)

    def close_due(self, t: int, dbg: Optional[torch.Tensor] = None) -> int:
        """Close every sequence whose window ends with token t; returns how many."""
        p = t % self.period
        n = self._close_n[p]
        if n == 0:
            return 0
        if n == self.dims.batch and dbg is None:
            lqk.window_close(self.dims, self.state, None, 0, None)
        else:
            ids = self._close_ids[self._close_at[p]:self._close_at[p] + n]
            lqk.window_close(self.dims, self.state, ids, n, dbg)
        return n

    def step(self, q, k, v, g, beta, o: Optional[torch.Tensor] = None, close: bool = True) -> torch.Tensor:
        """Token self.t on every head, then (close) the closes it makes due."""
        o = self.o if o is None else o
        n = self.fused_at(self.t) if close else -1
        if n >= 0:
            lqk.decode_close_at(self.dims, self.state, n, q, k, v, g, beta, o)
        else:
            self.decode(self.t, q, k, v, g, beta, o)
            if close:
                self.close_due(self.t)
        self.t += 1
        return o


def capture_tokens(decs, inputs, outs, t0: int, t1: int, overlap: bool = True) -> torch.cuda.CUDAGraph:
    """One HIP graph that advances a stack of layers, each with its own Decoder,
    through tokens t0..t1-1: per token the decode step of every layer in layer
    order, and the window closes due after it (as separate launches: the
    token's output comes from its decode launch on the capture stream, and
    only the close, which produces no output, moves to a side stream).

    inputs[l]: device token tensors of layer l with a leading token axis (q, k,
    v, g, beta); outs[l]: the output buffer of layer l. overlap=False closes
    every layer after the token's last decode. overlap=True forks the close of
    layer l onto a side stream as soon as layer l's decode is done, and makes
    only layer l's next decode wait for it: the closes (bound by the vector
    ALU) then run beside the other layers' decodes (bound by HBM). Both orders
    respect every dependency of the step, so they give the same results. All
    side streams are joined before the graph ends. Capturing runs nothing; the
    Decoders' own token counters are not used or changed."""
    L = len(decs)
    g = torch.cuda.CUDAGraph()
    sides = [torch.cuda.Stream() for _ in range(L)] if overlap else []
    pending = [None] * L
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream()
        for t in range(t0, t1):
            for l, dec in enumerate(decs):
                if pending[l] is not None:
                    cap.wait_event(pending[l])
                    pending[l] = None
                x = inputs[l]
                dec.decode(t, x["q"][t], x["k"][t], x["v"][t], x["g"][t], x["beta"][t], outs[l])
                if overlap and dec.closes_at(t):
                    ready = torch.cuda.Event()
                    ready.record(cap)
                    sides[l].wait_event(ready)
                    with torch.cuda.stream(sides[l]):
                        dec.close_due(t)
                    pending[l] = torch.cuda.Event()
                    pending[l].record(sides[l])
            if not overlap:
                for dec in decs:
                    dec.close_due(t)
        for ev in pending:
            if ev is not None:
                cap.wait_event(ev)
    return g

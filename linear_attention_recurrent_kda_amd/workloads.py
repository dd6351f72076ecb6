"""Seeded synthetic decode workloads for delta-rule linear attention.

This module only draws inputs: initial recurrent states with planted outlier
rows and columns, per-token queries, keys, values, decays and write
strengths, and the per-sequence window schedule. It contains none of the
method's arithmetic, so both the fp64 oracle tests and the HIP path can take
their inputs from here without sharing any computation.

Shapes follow the five decode workloads of the LeapQuant study (GDN scalar
decay and KDA per-channel decay, head dimension 32 or 128, window 16 or 32).
The pages give no data, only distributions, so every tensor is synthetic:

* q, k, v ~ N(0, 1); q and k are L2-normalised in fp32 (the usual
  normalisation in GDN/KDA layers). For bf16 activations the normalised fp32
  value is rounded to bf16 (round to nearest even) and both sides consume
  the rounded value.
* beta = sigmoid(N(0, 1)).
* GDN decay: g = log(alpha) with alpha = exp(-softplus(N(0,1)) * 0.05), or
  alpha ~ U(0.9, 1) for the Qwen-style workload.
* KDA decay: g[i] = -softplus(N(0,1)) * lam[h, i], lam ~ U(0.01, 0.2) fixed
  per (head, key channel).
* S_init ~ N(0, sigma) in the math layout [d_k][d_v] (row = key channel),
  with distinct outlier rows multiplied first and outlier columns second.

Random streams are independent per (workload, seed, sequence, quantity), so
any subset of sequences can be regenerated exactly and drawing in chunks of
steps gives the same values as drawing all steps at once.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

# quantity ids of the per-sequence random streams
_STATE, _Q, _K, _V, _G, _BETA, _OFFSET = range(7)


@dataclass(frozen=True)
class Workload:
    """One decode workload: shapes, window schedule and input distributions."""

    name: str
    config_id: int
    batch: int
    heads: int
    d_k: int
    d_v: int
    steps: int
    window: int            # W for every sequence (ignored when mixed_window)
    n_comp: int            # r compensators
    bits: int = 8
    kda: bool = False      # per-key-channel decay
    act_bf16: bool = False
    decay: str = "softplus"        # "softplus" (scaled by decay_scale) or "uniform" (alpha ~ U(0.9,1))
    decay_scale: float = 0.05
    kda_lam: tuple = (0.01, 0.2)
    state_sigma: float = 0.1
    out_rows: int = 2
    row_mult: float = 50.0
    out_cols: int = 1
    col_mult: float = 20.0
    staggered: bool = False        # random start offset 0..15 inside the first window
    mixed_window: bool = False     # W=16 for even sequences, 32 for odd
    smoothing: bool = True
    power_iters: int = 4
    warm_start: bool = False       # compensators start from the closing window's (a variant)
    seed: int = 0

    @property
    def w_max(self) -> int:
        return 32 if self.mixed_window else self.window

    @property
    def n_heads_total(self) -> int:
        return self.batch * self.heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # tiny GDN decode: 1 x 1 head, d=32, 64 steps, W=16, r=2, int8
    "tiny_gdn": Workload("tiny_gdn", 1, batch=1, heads=1, d_k=32, d_v=32, steps=64,
                         window=16, n_comp=2),
    # Qwen-style GDN decode: 64 x 32 heads, d=128, 256 steps, W=16, r=4, bf16 activations
    "qwen_gdn": Workload("qwen_gdn", 2, batch=64, heads=32, d_k=128, d_v=128, steps=256,
                         window=16, n_comp=4, act_bf16=True, decay="uniform",
                         state_sigma=0.05, out_rows=4, row_mult=100.0, out_cols=2,
                         col_mult=30.0),
    # serving-scale GDN decode: 256 x 32 heads, 512 steps
    "serving_gdn": Workload("serving_gdn", 3, batch=256, heads=32, d_k=128, d_v=128,
                            steps=512, window=16, n_comp=4),
    # KDA per-channel decay: 128 x 32 heads, 256 steps, int4 packed (also run at int8)
    "kda_int4": Workload("kda_int4", 4, batch=128, heads=32, d_k=128, d_v=128, steps=256,
                         window=16, n_comp=4, bits=4, kda=True),
    # prefix-cache decode mix: 512 x 48 heads, 1024 steps, staggered W=16/32 windows
    "prefix_mix": Workload("prefix_mix", 5, batch=512, heads=48, d_k=128, d_v=128,
                           steps=1024, window=16, n_comp=4, staggered=True,
                           mixed_window=True),
}


def _rng(wl: Workload, b: int, quantity: int) -> np.random.Generator:
    return np.random.default_rng([wl.config_id, wl.seed, b, quantity])


def kda_lambda(wl: Workload) -> np.ndarray:
    """Per (head, key channel) decay rates lam ~ U(lo, hi), shared by all sequences. [H, d_k] fp32."""
    rng = np.random.default_rng([wl.config_id, wl.seed, 10 ** 6])
    lo, hi = wl.kda_lam
    return rng.uniform(lo, hi, size=(wl.heads, wl.d_k)).astype(np.float32)


def window_lengths(wl: Workload) -> np.ndarray:
    """Per-sequence window length W_b. [B] int32."""
    if wl.mixed_window:
        return np.where(np.arange(wl.batch) % 2 == 0, 16, 32).astype(np.int32)
    return np.full(wl.batch, wl.window, np.int32)


def window_offsets(wl: Workload) -> np.ndarray:
    """Per-sequence start position inside the first window (0 unless staggered). [B] int32."""
    if not wl.staggered:
        return np.zeros(wl.batch, np.int32)
    return np.array([int(_rng(wl, b, _OFFSET).integers(0, 16)) for b in range(wl.batch)], np.int32)


def initial_state(wl: Workload, b: int) -> np.ndarray:
    """Initial fp32 state of every head of sequence b, math layout [H][d_k][d_v]."""
    rng = _rng(wl, b, _STATE)
    S = rng.normal(0.0, wl.state_sigma, size=(wl.heads, wl.d_k, wl.d_v)).astype(np.float32)
    for h in range(wl.heads):
        rows = rng.choice(wl.d_k, size=wl.out_rows, replace=False)
        cols = rng.choice(wl.d_v, size=wl.out_cols, replace=False)
        S[h, rows, :] *= np.float32(wl.row_mult)
        S[h, :, cols] *= np.float32(wl.col_mult)
    return S


def initial_states(wl: Workload, seqs: Iterable[int]) -> np.ndarray:
    """[len(seqs)][H][d_k][d_v] fp32."""
    return np.stack([initial_state(wl, b) for b in seqs])


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even); returns the raw uint16 bits."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((bits >> 16) & 1)
    return ((bits + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def _l2n(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


class TokenStream:
    """Per-sequence token inputs, drawn in chunks of steps.

    `next(n)` returns the next n steps for the listed sequences as a dict of
    arrays with leading axes [n][S][H]:
      q, k, v : fp32 values that both sides compute with (bf16-rounded when the
                workload has bf16 activations)
      q16, k16, v16 : raw bf16 bits (uint16), only for bf16 workloads
      g     : log-decay, [n][S][H] (GDN) or [n][S][H][d_k] (KDA), fp32
      beta  : [n][S][H] fp32
    """

    def __init__(self, wl: Workload, seqs: Optional[Sequence[int]] = None):
        self.wl = wl
        self.seqs: List[int] = list(range(wl.batch)) if seqs is None else list(seqs)
        self._r = {b: [_rng(wl, b, qq) for qq in (_Q, _K, _V, _G, _BETA)] for b in self.seqs}
        self._lam = kda_lambda(wl) if wl.kda else None
        self.t = 0

    def next(self, n: int) -> Dict[str, np.ndarray]:
        wl = self.wl
        H, dk, dv = wl.heads, wl.d_k, wl.d_v
        S = len(self.seqs)
        q = np.empty((n, S, H, dk), np.float32)
        k = np.empty((n, S, H, dk), np.float32)
        v = np.empty((n, S, H, dv), np.float32)
        gshape = (n, S, H, dk) if wl.kda else (n, S, H)
        g = np.empty(gshape, np.float32)
        beta = np.empty((n, S, H), np.float32)
        for si, b in enumerate(self.seqs):
            rq, rk, rv, rg, rb = self._r[b]
            q[:, si] = _l2n(rq.standard_normal((n, H, dk), dtype=np.float32))
            k[:, si] = _l2n(rk.standard_normal((n, H, dk), dtype=np.float32))
            v[:, si] = rv.standard_normal((n, H, dv), dtype=np.float32)
            if wl.kda:
                x = rg.standard_normal((n, H, dk), dtype=np.float32)
                g[:, si] = (-_softplus(x) * self._lam[None].astype(np.float64)).astype(np.float32)
            elif wl.decay == "uniform":
                alpha = rg.uniform(0.9, 1.0, size=(n, H))
                g[:, si] = np.log(alpha).astype(np.float32)
            else:
                x = rg.standard_normal((n, H), dtype=np.float32)
                g[:, si] = (-_softplus(x) * wl.decay_scale).astype(np.float32)
            beta[:, si] = _sigmoid(rb.standard_normal((n, H), dtype=np.float32)).astype(np.float32)
        out = {"g": g, "beta": beta}
        if wl.act_bf16:
            for name, arr in (("q", q), ("k", k), ("v", v)):
                bits = round_to_bf16(arr)
                out[name + "16"] = bits
                out[name] = bf16_to_f32(bits)
        else:
            out.update(q=q, k=k, v=v)
        self.t += n
        return out



def device_tokens(wl: Workload, steps: int, seed: int = 0, device="cuda"):
    """Token inputs for throughput runs, drawn on the device with torch's seeded
    generator: the same distributions as TokenStream (a different random
    stream), laid out [steps][B*H][...] exactly as the decode kernels read one
    step. Values are never compared with the oracle; parity runs use
    TokenStream."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(1_000_003 * wl.config_id + seed)
    BH, dk, dv = wl.batch * wl.heads, wl.d_k, wl.d_v
    f32 = dict(device=device, dtype=torch.float32, generator=gen)

    def unit(x):
        return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)

    q = unit(torch.randn((steps, BH, dk), **f32))
    k = unit(torch.randn((steps, BH, dk), **f32))
    v = torch.randn((steps, BH, dv), **f32)
    if wl.kda:
        lam = torch.from_numpy(kda_lambda(wl)).to(device)               # [H][d_k]
        lam = lam.repeat(wl.batch, 1)                                    # [B*H][d_k]
        g = -torch.nn.functional.softplus(torch.randn((steps, BH, dk), **f32)) * lam
    elif wl.decay == "uniform":
        g = torch.log(0.9 + 0.1 * torch.rand((steps, BH), **f32))
    else:
        g = -torch.nn.functional.softplus(torch.randn((steps, BH), **f32)) * wl.decay_scale
    beta = torch.sigmoid(torch.randn((steps, BH), **f32))
    if wl.act_bf16:
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), g=g.contiguous(), beta=beta.contiguous())

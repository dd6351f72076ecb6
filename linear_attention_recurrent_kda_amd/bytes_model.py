"""Algorithmic HBM bytes of the LeapQuant decode path, per head (one head =
one (sequence, head) pair). Each tensor the method needs is counted once per
launch: what the kernel must read and write, not what it happens to move.

decode step at window position n (n tokens already buffered):
    codes d_k*d_v*bits/8 + scales 4(d_k + d_v) + compensators 4r(d_k + d_v)
  + buffer read n*E + activations act*(2 d_k + d_v) + decay 4*g_len + beta 4
  + output 4 d_v + buffer append E,        E = act*d_k + 4(d_v + g_len)
(a buffered token's key is kept at the activation width: bf16 activations give
bf16 keys, exactly; its value u and G are fp32)
window close after n tokens:
    read codes + scales + compensators + n*E, write codes + scales + compensators
the window's last token taken inside its close (n tokens buffered before it):
    the close over the n buffered rows + activations, decay, beta + output
FP32-state baseline step:
    state read + write 2*4*d_k*d_v + activations + decay + beta + output
g_len = 1 for GDN (scalar decay), d_k for KDA (per-key-channel decay).
"""
from __future__ import annotations


def _parts(d: int, r: int, bits: int, kda: bool, bf16: bool):
    g_len = d if kda else 1
    act = 2 if bf16 else 4
    E = act * d + 4 * (d + g_len)
    lowbit = d * d * bits // 8 + 4 * 2 * d + 4 * r * 2 * d
    acts = act * 3 * d + 4 * g_len + 4
    return g_len, E, lowbit, acts


def step_bytes(d: int, r: int, bits: int, kda: bool, bf16: bool, n: int) -> int:
    g_len, E, lowbit, acts = _parts(d, r, bits, kda, bf16)
    return lowbit + n * E + acts + 4 * d + E


def close_bytes(d: int, r: int, bits: int, kda: bool, bf16: bool, n: int) -> int:
    g_len, E, lowbit, acts = _parts(d, r, bits, kda, bf16)
    return 2 * lowbit + n * E


def fused_bytes(d: int, r: int, bits: int, kda: bool, bf16: bool, n: int) -> int:
    g_len, E, lowbit, acts = _parts(d, r, bits, kda, bf16)
    return 2 * lowbit + n * E + acts + 4 * d


def fp32_step_bytes(d: int, kda: bool, bf16: bool) -> int:
    g_len = d if kda else 1
    act = 2 if bf16 else 4
    return 2 * 4 * d * d + act * 3 * d + 4 * g_len + 4 + 4 * d


def window_avg_step_bytes(d: int, r: int, bits: int, kda: bool, bf16: bool, W: int) -> float:
    return sum(step_bytes(d, r, bits, kda, bf16, n) for n in range(W)) / W

"""Host logic of bench.py's schedule: which steps a launch takes inside the
window close, and how the plan splits decode graphs around them (graph
capture stubbed out; no GPU)."""
import types

import numpy as np

import bench
from linear_attention_recurrent_kda_amd import bytes_model as bm


class _Stub(bench.Graphs):
    def decode(self, a, b):
        return None if b <= a else ("decode", a, b)

    def close(self, t):
        return ("close", t, self.fused_at(t)) if len(self.closes[t]) else None


def _graphs(win_len, win_off, total, fuse=True, batch=None):
    closes, ns = bench.schedule(np.asarray(win_len), np.asarray(win_off), total)
    dims = types.SimpleNamespace(batch=len(win_len) if batch is None else batch)
    return _Stub(dims, [None], [None], [None], closes, None, None, ns=ns, fuse=fuse), closes, ns


def test_aligned_windows_take_the_last_token_inside_the_close():
    gr, closes, ns = _graphs([16] * 4, [0] * 4, 64)
    assert [gr.fused_at(t) for t in range(32)] == [-1] * 15 + [15] + [-1] * 15 + [15]
    plan = gr.plan(5, 40)
    assert [(a, b, f) for (a, b, _d, _c, f) in plan] == [(5, 16, True), (16, 32, True), (32, 40, False)]
    assert plan[0][2] == ("decode", 5, 15) and plan[0][3] == ("close", 15, 15)
    assert plan[2][2] == ("decode", 32, 40) and plan[2][3] is None
    # every step of [5, 40) is taken once: by a decode launch or inside a close
    taken = [t for (_a, _b, d, _c, _f) in plan if d for t in range(d[1], d[2])]
    taken += [c[1] for (_a, _b, _d, c, f) in plan if f]
    assert sorted(taken) == list(range(5, 40))


def test_window_of_one_token_leaves_no_decode_graph():
    gr, _, _ = _graphs([1] * 3, [0] * 3, 4)
    plan = gr.plan(0, 4)
    assert all(d is None and f for (_a, _b, d, _c, f) in plan)


def test_staggered_or_partial_closes_keep_separate_launches():
    gr, closes, _ = _graphs([16, 16, 32, 32], [0, 3, 0, 7], 64)      # staggered, two window lengths
    assert all(gr.fused_at(t) == -1 for t in range(64))
    gr, closes, _ = _graphs([16, 32], [0, 0], 64)                    # aligned starts, different lengths
    assert gr.fused_at(15) == -1                                     # only sequence 0 closes
    assert len(closes[31]) == 2 and gr.fused_at(31) == -1            # both close, at positions 15 and 31
    gr, _, _ = _graphs([16] * 4, [0] * 4, 32, fuse=False)
    assert all(gr.fused_at(t) == -1 for t in range(32))


def test_fused_bytes_count_the_token_once():
    """The fused launch reads the close's bytes over the n buffered rows plus
    the token's activations and writes its output; against a decode launch
    plus a close of n + 1 rows it saves one pass over the low-bit state, the
    n buffered rows and the appended row (written and read back). A buffered
    token's key is kept at the activation width (bf16 activations: 2 bytes)."""
    d, r = 128, 4
    for bits in (8, 6, 4):
        for kda in (False, True):
            for bf16 in (False, True):
                for n in (0, 7, 15):
                    E = (2 if bf16 else 4) * d + 4 * (d + (d if kda else 1))
                    lowbit = d * d * bits // 8 + 8 * d + 8 * r * d
                    saved = (bm.step_bytes(d, r, bits, kda, bf16, n) + bm.close_bytes(d, r, bits, kda, bf16, n + 1)
                             - bm.fused_bytes(d, r, bits, kda, bf16, n))
                    assert saved == lowbit + n * E + 2 * E

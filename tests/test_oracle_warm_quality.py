"""Output error of warm-started compensators against the exact recurrence
(oracle only). A warm start is a variant, not on the pages: its claim is
that starting each close's power method from the closing window's
compensator values needs fewer iterations for the same output error. The
reference here is the plain recurrence with no quantization and no
compensators; the error is the mean over tokens of the relative L2 of o."""
import numpy as np
import pytest

from linear_attention_recurrent_kda_amd import workloads as wk
from oracle import leapquant_oracle as lq
from tests import gpu_helpers as gh


def _errors(name, n_seq, steps, runs):
    wl = wk.WORKLOADS[name]
    seqs = list(range(n_seq))
    S0 = wk.initial_states(wl, seqs).reshape(-1, wl.d_k, wl.d_v).astype(np.float64)
    toks = gh.flat_steps(wk.TokenStream(wl, seqs).next(steps))
    wlen = np.repeat(wk.window_lengths(wl)[seqs], wl.heads)
    woff = np.repeat(wk.window_offsets(wl)[seqs], wl.heads)
    exact = lq.run_dense(S0, toks, wlen, woff, r=0, T=1, bits=wl.bits, quantize=False)["o"]
    out = {}
    for T, warm in runs:
        o = lq.run_dense(S0, toks, wlen, woff, r=wl.n_comp, T=T, bits=wl.bits, warm_start=warm)["o"]
        out[(T, warm)] = float(np.mean([np.linalg.norm(o[t] - exact[t]) / np.linalg.norm(exact[t])
                                        for t in range(steps)]))
    return out


@pytest.mark.parametrize("name,n_seq,steps", [("qwen_gdn", 2, 128), ("kda_int4", 1, 128)])
def test_warm_start_needs_fewer_iterations(name, n_seq, steps):
    e = _errors(name, n_seq, steps, [(4, False), (2, False), (1, False), (2, True), (1, True)])
    print(name, {f"T={T}{' warm' if w else ''}": f"{v:.4e}" for (T, w), v in e.items()})
    # one warm iteration beats one cold one; two warm ones come close to four cold ones
    assert e[(1, True)] < e[(1, False)]
    assert e[(2, True)] <= 1.05 * e[(4, False)]
    assert e[(2, True)] <= e[(2, False)] * 1.01

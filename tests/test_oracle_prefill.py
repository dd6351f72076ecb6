"""Pins of the oracle's prefill handoff (CPU only): the prompt runs the exact
recurrence token by token, and its final state is encoded once.

Pinned against closed forms over a whole prompt (pure decay accumulates, a
last write with beta = 1 and a unit key is memorised, the token order
matters), against the explicit GDN / KDA matrix forms applied token after
token, and against the encode's own reconstruction invariant."""
import numpy as np
import pytest

from oracle import leapquant_oracle as lq
from tests.oracle_inputs import unit


def _toks(rng, L, N, d, kda, beta=None):
    out = []
    for _ in range(L):
        g = -0.3 * rng.random((N, d) if kda else N)
        out.append(dict(q=unit(rng.standard_normal((N, d))), k=unit(rng.standard_normal((N, d))),
                        v=rng.standard_normal((N, d)), g=g,
                        beta=np.full(N, beta) if beta is not None else rng.random(N)))
    return out


@pytest.mark.parametrize("kda", [False, True])
def test_pure_decay_accumulates(kda):
    """beta = 0: S_L = exp(sum_t g_t) (.)_rows S_0 and o_t = (exp(G_t) (.) S_0)^T q_t."""
    rng = np.random.default_rng(1)
    N, d, L = 3, 4, 7
    S0 = rng.standard_normal((N, d, d))
    toks = _toks(rng, L, N, d, kda, beta=0.0)
    S, outs = lq.prefill(S0, toks)
    G = np.zeros((N, d) if kda else N)
    for t, tk in enumerate(toks):
        G = G + tk["g"]
        St = S0 * (np.exp(G)[:, :, None] if kda else np.exp(G)[:, None, None])
        np.testing.assert_allclose(outs[t], np.einsum("nij,ni->nj", St, tk["q"]), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S, St, rtol=1e-13, atol=1e-13)


def test_last_write_is_memorised_and_order_matters():
    rng = np.random.default_rng(2)
    N, d, L = 4, 4, 6
    S0 = rng.standard_normal((N, d, d))
    toks = _toks(rng, L, N, d, False)
    toks[-1]["beta"] = np.ones(N)
    S, _ = lq.prefill(S0, toks)
    np.testing.assert_allclose(np.einsum("nij,ni->nj", S, toks[-1]["k"]), toks[-1]["v"], rtol=1e-12, atol=1e-12)
    S_rev, _ = lq.prefill(S0, toks[::-1])
    assert np.abs(S_rev - S).max() > 1e-3


@pytest.mark.parametrize("kda", [False, True])
def test_matches_matrix_form_token_by_token(kda):
    rng = np.random.default_rng(3)
    N, d, L = 2, 4, 5
    I = np.eye(d)
    S0 = rng.standard_normal((N, d, d))
    toks = _toks(rng, L, N, d, kda)
    S_ref = S0.copy()
    outs_ref = []
    for tk in toks:
        for n in range(N):
            k, v, b = tk["k"][n], tk["v"][n], tk["beta"][n]
            A = np.diag(np.exp(tk["g"][n])) if kda else np.exp(tk["g"][n]) * I
            S_ref[n] = (I - b * np.outer(k, k)) @ A @ S_ref[n] + b * np.outer(k, v)
        outs_ref.append(np.einsum("nij,ni->nj", S_ref, tk["q"]))
    S, outs = lq.prefill(S0, toks)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)
    for a, b in zip(outs, outs_ref):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_handoff_encodes_the_final_state():
    rng = np.random.default_rng(4)
    N, d, L = 3, 8, 9
    S0 = rng.standard_normal((N, d, d))
    toks = _toks(rng, L, N, d, False)
    enc, S, outs = lq.prefill_handoff(S0, toks, r=2, T=4, bits=8)
    assert len(outs) == L
    # compensators plus the unquantised residual rebuild the prompt's final state
    rebuilt = np.einsum("nli,nlj->nij", enc.comp_k, enc.comp_u) + enc.resid
    np.testing.assert_allclose(rebuilt, S, rtol=1e-12, atol=1e-12)
    # and the quantised window-start state is within the quantiser's bound of it
    err = np.abs(lq.decode(enc) - S)
    bound = enc.s[:, :, None] * enc.c[:, None, :] / 2 + 1e-12
    assert np.all(err <= bound)

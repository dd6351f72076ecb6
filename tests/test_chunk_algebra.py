"""The chunked form of the prompt recurrence, written out in fp64 NumPy and
checked against the oracle's token-by-token prefill (CPU only).

At d_k = 128 the HIP prefill evaluates the prompt in chunks: within a chunk
with start state S0 and cumulative log-decays G_t (through token t, per key
channel for KDA), (alpha_t S_{t-1})^T k_t, o_t and the end state expand into
S0 products plus sums over the chunk's earlier tokens weighted by
e^{G_t - G_s}, and the u_t solve a unit lower-triangular system. This test
states that algebra independently of the kernels and shows it is the same
recurrence: outputs and states agree with the oracle to rounding, for GDN and
KDA, over full and ragged chunks."""
import numpy as np
import pytest

from oracle import leapquant_oracle as lq
from tests.oracle_inputs import unit


def _toks(rng, L, N, d, kda):
    out = []
    for _ in range(L):
        g = -0.4 * rng.random((N, d) if kda else N)
        out.append(dict(q=unit(rng.standard_normal((N, d))), k=unit(rng.standard_normal((N, d))),
                        v=rng.standard_normal((N, d)), g=g, beta=rng.random(N)))
    return out


def _chunked_head(S0, toks, h, C, kda):
    """One head, chunks of C tokens: returns (S_end, outputs)."""
    S = S0.copy()
    d = S.shape[0]
    outs = []
    for c0 in range(0, len(toks), C):
        ch = toks[c0:c0 + C]
        n = len(ch)
        K = np.stack([t["k"][h] for t in ch])
        Q = np.stack([t["q"][h] for t in ch])
        V = np.stack([t["v"][h] for t in ch])
        beta = np.array([t["beta"][h] for t in ch])
        g = np.stack([np.broadcast_to(t["g"][h], (d,)) for t in ch])  # [n][d_k]
        G = np.cumsum(g, axis=0)
        E = np.exp(G)  # e^{G_t} per channel
        A = np.zeros((n, n))
        B = np.zeros((n, n))
        for t in range(n):
            for s in range(t + 1):
                f = np.exp(G[t] - G[s])
                B[t, s] = np.sum(Q[t] * K[s] * f)
                if s < t:
                    A[t, s] = np.sum(K[t] * K[s] * f)
        R = beta[:, None] * (V - (K * E) @ S)
        U = np.zeros_like(R)
        for t in range(n):
            U[t] = R[t] - beta[t] * (A[t, :t] @ U[:t])
        O = (Q * E) @ S + B @ U
        outs.extend(O)
        S = E[-1][:, None] * S + (K * np.exp(G[-1] - G)).T @ U
    return S, outs


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("L,C", [(16, 4), (11, 4), (37, 16), (5, 16)])
def test_chunked_form_equals_recurrence(kda, L, C):
    rng = np.random.default_rng(7 + L + C + kda)
    N, d = 3, 8
    S0 = rng.standard_normal((N, d, d))
    toks = _toks(rng, L, N, d, kda)
    S_ref, outs_ref = lq.prefill(S0, toks)
    for h in range(N):
        S_h, outs_h = _chunked_head(S0[h], toks, h, C, kda)
        assert np.allclose(S_h, S_ref[h], rtol=1e-10, atol=1e-12)
        for t in range(L):
            assert np.allclose(outs_h[t], outs_ref[t][h], rtol=1e-10, atol=1e-12)


def test_chunked_form_with_an_underflowing_decay():
    """A token whose decay underflows: every factor is an exponent <= 0, so the
    chunked form stays finite and still matches."""
    rng = np.random.default_rng(3)
    N, d, L = 2, 8, 12
    S0 = rng.standard_normal((N, d, d))
    toks = _toks(rng, L, N, d, True)
    toks[6]["g"] = np.full((N, d), -800.0)
    S_ref, outs_ref = lq.prefill(S0, toks)
    for h in range(N):
        S_h, outs_h = _chunked_head(S0[h], toks, h, 4, True)
        assert np.all(np.isfinite(S_h))
        assert np.allclose(S_h, S_ref[h], rtol=1e-10, atol=1e-12)
        for t in range(L):
            assert np.allclose(outs_h[t], outs_ref[t][h], rtol=1e-10, atol=1e-12)

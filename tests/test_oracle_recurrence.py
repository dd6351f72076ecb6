"""Pins of the oracle's exact GDN / KDA recurrence (CPU only).

Each check compares against something other than the oracle's own formula: a
hand-worked example, the explicit matrix forms of the gated delta rule, and
closed forms (pure decay, delta-rule memorisation, KDA with equal channel
decays reducing to GDN).
"""
import numpy as np
import pytest

from oracle import leapquant_oracle as lq
from tests.oracle_inputs import unit


def test_hand_worked_2x2_gdn_and_kda():
    # S rows are key channels. alpha = 1/2, beta = 1/2, k = e_0, v = (2, 4), q = e_1.
    # GDN by hand: S' = S/2 = [[.5,1],[1.5,2]]; S'^T k = (.5, 1); u = (.75, 1.5);
    # S_t = [[1.25, 2.5],[1.5, 2]]; o = S_t^T q = (1.5, 2).
    S = np.array([[[1.0, 2.0], [3.0, 4.0]]])
    q = np.array([[0.0, 1.0]])
    k = np.array([[1.0, 0.0]])
    v = np.array([[2.0, 4.0]])
    beta = np.array([0.5])
    St, o, u = lq.exact_step(S, q, k, v, np.log([0.5]), beta)
    np.testing.assert_allclose(St[0], [[1.25, 2.5], [1.5, 2.0]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0], [1.5, 2.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(u[0], [0.75, 1.5], rtol=0, atol=1e-15)
    # KDA with alpha = (1/2, 1/4): S' = [[.5,1],[.75,1]]; u = (.75, 1.5);
    # S_t = [[1.25, 2.5],[.75, 1]]; o = (.75, 1).
    St, o, u = lq.exact_step(S, q, k, v, np.log([[0.5, 0.25]]), beta)
    np.testing.assert_allclose(St[0], [[1.25, 2.5], [0.75, 1.0]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0], [0.75, 1.0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("kda", [False, True])
def test_matches_explicit_matrix_form_4x4(kda):
    rng = np.random.default_rng(11)
    N, d = 6, 4
    I = np.eye(d)
    for _ in range(5):
        S = rng.standard_normal((N, d, d))
        k = unit(rng.standard_normal((N, d)))
        q = rng.standard_normal((N, d))
        v = rng.standard_normal((N, d))
        beta = rng.uniform(0, 1, N)
        g = -rng.uniform(0, 1, (N, d) if kda else N)
        St, o, u = lq.exact_step(S, q, k, v, g, beta)
        for n in range(N):
            P = I - beta[n] * np.outer(k[n], k[n])
            if kda:
                ref = P @ np.diag(np.exp(g[n])) @ S[n] + beta[n] * np.outer(k[n], v[n])
            else:
                ref = np.exp(g[n]) * (P @ S[n]) + beta[n] * np.outer(k[n], v[n])
            np.testing.assert_allclose(St[n], ref, rtol=0, atol=1e-14)
            np.testing.assert_allclose(o[n], ref.T @ q[n], rtol=0, atol=1e-14)


@pytest.mark.parametrize("kda", [False, True])
def test_beta_zero_is_pure_decay(kda):
    rng = np.random.default_rng(3)
    N, dk, dv, T = 3, 5, 7, 9
    S0 = rng.standard_normal((N, dk, dv))
    S = S0.copy()
    G = np.zeros((N, dk) if kda else N)
    for _ in range(T):
        g = -rng.uniform(0, 0.3, G.shape)
        q = rng.standard_normal((N, dk))
        S, o, _ = lq.exact_step(S, q, unit(rng.standard_normal((N, dk))), rng.standard_normal((N, dv)), g,
                                np.zeros(N))
        G = G + g
        ref = S0 * (np.exp(G)[:, :, None] if kda else np.exp(G)[:, None, None])
        np.testing.assert_allclose(S, ref, rtol=1e-13, atol=0)
        np.testing.assert_allclose(o, np.einsum("nij,ni->nj", ref, q), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("kda", [False, True])
def test_beta_one_unit_key_memorises_value(kda):
    rng = np.random.default_rng(5)
    N, dk, dv = 4, 8, 6
    S = rng.standard_normal((N, dk, dv))
    for _ in range(6):
        k = unit(rng.standard_normal((N, dk)))
        v = rng.standard_normal((N, dv))
        g = -rng.uniform(0, 0.5, (N, dk) if kda else N)
        S, o, _ = lq.exact_step(S, k, k, v, g, np.ones(N))
        # S_t^T k_t = v_t exactly, so reading with q = k returns v
        np.testing.assert_allclose(np.einsum("nij,ni->nj", S, k), v, rtol=0, atol=1e-13)
        np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)


def test_kda_with_equal_channel_decays_is_gdn():
    rng = np.random.default_rng(9)
    N, dk, dv = 3, 6, 5
    S1 = rng.standard_normal((N, dk, dv))
    S2 = S1.copy()
    for _ in range(8):
        q, k = rng.standard_normal((N, dk)), unit(rng.standard_normal((N, dk)))
        v, beta = rng.standard_normal((N, dv)), rng.uniform(0, 1, N)
        g = -rng.uniform(0, 0.4, N)
        S1, o1, u1 = lq.exact_step(S1, q, k, v, g, beta)
        S2, o2, u2 = lq.exact_step(S2, q, k, v, np.repeat(g[:, None], dk, axis=1), beta)
        np.testing.assert_array_equal(S1, S2)
        np.testing.assert_array_equal(o1, o2)

"""Pins of the oracle's window-close encoder (CPU only): start vectors,
compensator extraction, smoothing and quantisation.

Pinned against: published SplitMix64 outputs (tests/golden), exact
reconstruction and orthogonality invariants, Pythagoras for deflation, the
rank-one closed form, numpy.linalg.svd in the converged limit, and an
exhaustive nearest-code search on 4x4 residuals.
"""
import os

import numpy as np
import pytest

from oracle import leapquant_oracle as lq
from tests.oracle_inputs import planted_state

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_outputs():
    n_lines = 0
    with open(os.path.join(GOLDEN, "splitmix64.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            seed, *outs = (int(x) for x in line.split())
            assert [lq.splitmix64(i + 1, seed) for i in range(len(outs))] == outs
            n_lines += 1
    assert n_lines == 3


def test_start_vectors_are_exact_odd_multiples():
    v0 = lq.start_vectors(4, 128)
    m = v0 * 2.0 ** 23
    assert np.all(np.abs(v0) < 1.0)
    assert np.array_equal(m, np.round(m)) and np.all(np.round(m) % 2 != 0)
    assert np.array_equal(v0.astype(np.float32).astype(np.float64), v0)
    # entry (l, j) comes from output l*d_v + j + 1: spot-check two entries
    assert v0[0, 0] == ((2 * (lq.splitmix64(1) >> 41) + 1) - 2 ** 23) / 2 ** 23
    assert v0[3, 127] == ((2 * (lq.splitmix64(3 * 128 + 128) >> 41) + 1) - 2 ** 23) / 2 ** 23


def _states():
    rng = np.random.default_rng(1)
    yield planted_state(rng, 8, 32, 32)
    yield planted_state(rng, 4, 128, 128, sigma=0.05, rows=4, rmul=100.0, cols=2, cmul=30.0)


@pytest.mark.parametrize("r", [1, 2, 4])
def test_compensators_plus_residual_reconstruct_state(r):
    for S in _states():
        ck, cu, R = lq.extract_compensators(S, r, 4)
        rec = np.einsum("nli,nlj->nij", ck, cu) + R
        assert np.linalg.norm(rec - S) / np.linalg.norm(S) <= 1e-12
        # unit, mutually orthogonal keys
        gram = np.einsum("nli,nmi->nlm", ck, ck)
        np.testing.assert_allclose(gram, np.broadcast_to(np.eye(r), gram.shape), rtol=0, atol=1e-12)


def test_deflation_obeys_pythagoras():
    for S in _states():
        M = S.copy()
        for r in range(1, 5):
            ck, cu, R = lq.extract_compensators(S, r, 4)
            prev = np.sum(M ** 2, axis=(1, 2))
            now = np.sum(R ** 2, axis=(1, 2))
            np.testing.assert_allclose(now, prev - np.sum(cu[:, r - 1] ** 2, axis=1), rtol=1e-10)
            M = R


def test_rank_one_state_is_captured_by_one_compensator():
    rng = np.random.default_rng(2)
    a, b = rng.standard_normal((3, 16)), rng.standard_normal((3, 12))
    S = a[:, :, None] * b[:, None, :]
    for T in (1, 4):
        ck, cu, R = lq.extract_compensators(S, 1, T)
        an = a / np.linalg.norm(a, axis=1, keepdims=True)
        assert np.allclose(np.abs(np.sum(ck[:, 0] * an, axis=1)), 1.0, atol=1e-12)
        assert np.max(np.abs(R)) <= 1e-12 * np.max(np.abs(S))


def test_converged_power_method_matches_svd():
    rng = np.random.default_rng(3)
    d = 24
    U, _ = np.linalg.qr(rng.standard_normal((d, d)))
    V, _ = np.linalg.qr(rng.standard_normal((d, d)))
    sig = np.array([10.0, 5.0, 2.5, 1.25] + [0.1] * (d - 4))
    S = (U * sig) @ V.T
    ck, cu, R = lq.extract_compensators(S[None], 4, 200)
    Us, ss, _ = np.linalg.svd(S)
    for l in range(4):
        assert abs(abs(ck[0, l] @ Us[:, l]) - 1.0) <= 1e-10
        assert abs(np.linalg.norm(cu[0, l]) - ss[l]) <= 1e-10 * ss[0]


def test_zero_state_is_degenerate_and_exact():
    S = np.zeros((2, 8, 8))
    e = lq.encode(S, 2, 4, 8)
    assert np.all(e.comp_k == 0) and np.all(e.comp_u == 0)
    assert np.all(e.s == 1.0) and np.all(e.c == 0.0) and np.all(e.codes == 0)
    assert np.all(lq.decode(e) == 0.0)


def test_nonfinite_head_does_not_touch_other_heads():
    rng = np.random.default_rng(4)
    S = planted_state(rng, 3, 8, 8)
    bad = S.copy()
    bad[1, 2, 3] = np.nan
    e1, e2 = lq.encode(S, 2, 4, 8), lq.encode(bad, 2, 4, 8)
    for n in (0, 2):
        assert np.array_equal(e1.codes[n], e2.codes[n]) and np.array_equal(e1.comp_u[n], e2.comp_u[n])
    assert np.all(e2.comp_k[1] == 0)


def _nearest_code(x, Q):
    """Exhaustive search over all 2Q+1 codes, ties to the even code."""
    best, bd = None, None
    for code in range(-Q, Q + 1):
        d = abs(x - code)
        if bd is None or d < bd or (d == bd and code % 2 == 0):
            best, bd = code, d
    return best


@pytest.mark.parametrize("bits", [8, 6, 4])
@pytest.mark.parametrize("smoothing", [True, False])
def test_quantiser_brute_force_4x4(bits, smoothing):
    # symmetric b-bit codes: the largest magnitude a signed b-bit integer
    # holds on both sides of zero
    Q = 2 ** (bits - 1) - 1
    rng = np.random.default_rng(5 + bits)
    R = rng.standard_normal((20, 4, 4)) * rng.uniform(0.1, 10, (20, 4, 1))
    R[0, :, 1] = 0.0            # zero column
    R[1, 2, :] = 0.0            # zero row
    R[2] = np.array([[0.5, -1.0, 0.25, 2.0]] * 4) * 3.0
    # exact ties on the code grid: every row max is 1 (so s = 1) and column 0
    # has max Q/2^p, so c_0 = 2^-p and the other entries land on x.5 exactly
    p2 = 2.0 ** (bits - 1)
    R[3] = 0.0
    R[3, :, 3] = 1.0
    R[3, :, 0] = np.array([Q, 2.5, -3.5, 0.5]) / p2
    s, c, C = lq.smooth_quantize(R, bits, smoothing)
    for n in range(R.shape[0]):
        for i in range(4):
            row_max = max(abs(R[n, i, j]) for j in range(4))
            assert s[n, i] == ((row_max if row_max > 0 else 1.0) if smoothing else 1.0)
        for j in range(4):
            col = [R[n, i, j] / s[n, i] for i in range(4)]
            m = max(abs(x) for x in col)
            assert c[n, j] == m / Q
            for i in range(4):
                want = 0 if m == 0 else _nearest_code(col[i] / c[n, j], Q)
                assert C[n, i, j] == want, (n, i, j)
    # error bound and range
    err = np.abs(R - s[:, :, None] * C * c[:, None, :])
    assert np.all(err <= s[:, :, None] * c[:, None, :] / 2 * (1 + 1e-12))
    assert np.all(np.abs(C) <= Q)
    nz = np.max(np.abs(R), axis=1) > 0
    assert np.all(np.max(np.abs(C), axis=1)[nz] == Q)
    assert np.all(C[0, :, 1] == 0) and c[0, 1] == 0.0
    assert list(C[3, :, 0]) == [Q, 2, -4, 0]
    if smoothing:
        assert np.all(s[1, 2] == 1.0)


@pytest.mark.parametrize("smoothing", [True, False])
def test_quantiser_power_of_two_scaling(smoothing):
    rng = np.random.default_rng(6)
    R = planted_state(rng, 4, 16, 16)
    s, c, C = lq.smooth_quantize(R, 8, smoothing)
    for p in (-7, 3, 20):
        s2, c2, C2 = lq.smooth_quantize(R * 2.0 ** p, 8, smoothing)
        assert np.array_equal(C, C2)
        if smoothing:
            assert np.array_equal(s2, s * 2.0 ** p) and np.array_equal(c2, c)
        else:
            assert np.array_equal(s2, s) and np.array_equal(c2, c * 2.0 ** p)


def test_encode_is_deterministic():
    S = planted_state(np.random.default_rng(7), 3, 32, 32)
    e1, e2 = lq.encode(S, 2, 4, 8), lq.encode(S.copy(), 2, 4, 8)
    for f in ("comp_k", "comp_u", "s", "c", "codes", "resid"):
        assert np.array_equal(getattr(e1, f), getattr(e2, f))


def test_outlier_ratio_hand_computed():
    """max|X| / median|X| over all entries of each head, worked by hand.
    Head 0 (2 x 3): |X| sorted 0.5 1 2 3 4 12, median (2 + 3) / 2 = 2.5,
    max 12, ratio 4.8. Head 1: |X| sorted 1 1 1 1 1 9, median 1, ratio 9.
    A mean in place of the median gives 22.5 / 6 = 3.75 -> 3.2 for head 0;
    a per-row statistic, a statistic over heads or a signed max all differ."""
    X = np.array([[[1.0, -2.0, 0.5], [3.0, -12.0, 4.0]],
                  [[1.0, 1.0, -1.0], [-1.0, 9.0, 1.0]]])
    np.testing.assert_array_equal(lq.outlier_ratio(X), [4.8, 9.0])
    # an odd entry count: |X| = 1..9 (signs mixed), median 5, max 9
    Y = (np.arange(1, 10, dtype=np.float64) * np.array([1, -1, 1, 1, -1, 1, -1, 1, 1]))[None].reshape(1, 3, 3)
    np.testing.assert_array_equal(lq.outlier_ratio(Y), [9.0 / 5.0])
    # transposing a head does not change its ratio
    np.testing.assert_array_equal(lq.outlier_ratio(np.swapaxes(X, 1, 2)), [4.8, 9.0])


def test_outlier_ratio_drops_through_compensators_and_smoothing():
    """In kind with the pages' outlier-to-median example: planted outlier rows
    and columns are removed by the compensators, smoothing balances the rest."""
    S = planted_state(np.random.default_rng(8), 16, 32, 32)
    e = lq.encode(S, 2, 4, 8)
    r_S = np.median(lq.outlier_ratio(S))
    r_R = np.median(lq.outlier_ratio(e.resid))
    r_Rt = np.median(lq.outlier_ratio(e.resid / e.s[:, :, None]))
    assert r_S > 10 * r_R and r_R > r_Rt


def test_warm_start_from_exact_singular_vectors_gives_the_svd_in_one_step():
    """Started from the exact right singular vectors, one power step lands on
    the singular pairs, compensator after compensator (deflation removes each
    pair exactly): compare with numpy.linalg.svd."""
    rng = np.random.default_rng(21)
    N, d, r = 3, 12, 3
    U, _ = np.linalg.qr(rng.standard_normal((d, d)))
    V, _ = np.linalg.qr(rng.standard_normal((d, d)))
    sig = np.array([9.0, 5.0, 3.0] + [0.5] * (d - 3))
    S = np.stack([U @ np.diag(sig) @ V.T for _ in range(N)])
    _, sv, Vt = np.linalg.svd(S[0])
    start = np.repeat(Vt[None, :r, :], N, axis=0) * 3.0          # any positive scale
    ck, cu, R = lq.extract_compensators(S, r, T=1, start=start)
    for l in range(r):
        np.testing.assert_allclose(np.abs(ck[:, l] @ U[:, l]), 1.0, atol=1e-12)
        np.testing.assert_allclose(np.linalg.norm(cu[:, l], axis=1), sv[l], rtol=1e-12)
    # a cold start with one step is far from the singular vectors
    ck0, _, _ = lq.extract_compensators(S, r, T=1)
    assert np.abs(ck0[0, 0] @ U[:, 0]) < 0.999


def test_warm_start_falls_back_where_the_start_is_zero():
    rng = np.random.default_rng(22)
    S = rng.standard_normal((4, 8, 8))
    start = rng.standard_normal((4, 2, 8))
    start[1] = 0.0
    start[2, 1] = np.nan
    a = lq.extract_compensators(S, 2, 3, start)
    cold = lq.extract_compensators(S, 2, 3)
    np.testing.assert_array_equal(a[0][1], cold[0][1])           # head 1: fixed start vectors
    warm_only = lq.extract_compensators(S[2:3], 2, 3, start[2:3])
    np.testing.assert_array_equal(a[0][2], warm_only[0][0])
    assert not np.array_equal(a[0][0], cold[0][0])               # head 0 did start warm


def test_warm_windowed_dense_equals_buffered():
    """The plain definition and the buffered form agree with warm starts too."""
    from tests.oracle_inputs import random_tokens
    rng = np.random.default_rng(23)
    N, d, L = 3, 8, 20
    S0 = rng.standard_normal((N, d, d))
    toks = random_tokens(rng, L, N, d, d, kda=False)
    W = np.array([4, 5, 6])
    off = np.zeros(N, np.int64)
    a = lq.run_dense(S0, toks, W, off, r=2, T=1, warm_start=True)
    b = lq.run_buffered(S0, toks, W, off, w_max=6, r=2, T=1, warm_start=True)
    np.testing.assert_allclose(a["o"], b["o"], rtol=1e-9, atol=1e-9)
    c = lq.run_dense(S0, toks, W, off, r=2, T=1)
    assert not np.allclose(a["o"], c["o"], rtol=1e-12, atol=1e-12)  # the variant does change the closes

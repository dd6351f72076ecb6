"""FP64 CPU oracle for LeapQuant decoding of GDN / KDA recurrent states.

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with
the HIP path and imports nothing from it; both sides take their inputs from
the seeded workload generators.

Everything here is plain NumPy in float64, vectorised over a flat batch of N
heads (one head = one (sequence, head) pair). The recurrent state of a head
is S in R^{d_k x d_v} in the math layout: row i is a key channel, column j a
value channel.

Sources (the pages' titles):
  [abstract]  "LeapQuant: Efficient Linear Attention with Accurate Recurrent
              State Quantization", original abstract (robotpapers.com page).
  [article]   wink.run news article "Linear attention has to move state every
              token it generates; LeapQuant compresses it to 8-bit without
              losing accuracy", paragraphs on the three techniques.
  [GDN]       Gated Delta Networks (Yang, Kautz & Hatamizadeh, ICLR 2025),
              gated delta rule. The pages only name the model.
  [KDA]       Kimi Linear technical report (Moonshot AI, 2025), Kimi Delta
              Attention with per-channel gates. The pages only name it.
  [SplitMix64] Steele, Lea & Flood, "Fast splittable pseudorandom number
              generators", OOPSLA 2014.

Readings taken where the pages are silent are listed with each function.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Iterable, List, Optional

import numpy as np

QMAX = {8: 127, 6: 31, 4: 7}

# ---------------------------------------------------------------------------
# Power-method start vectors: SplitMix64 [SplitMix64], counter form.
# ---------------------------------------------------------------------------
_GOLDEN = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB
_M64 = (1 << 64) - 1


def splitmix64(n: int, seed: int = 0) -> int:
    """The n-th output (1-based) of SplitMix64 started from state `seed`.

    The state after n increments is seed + n * golden-gamma (mod 2^64); the
    output is that state passed through the published finaliser (xor-shift 30,
    multiply, xor-shift 27, multiply, xor-shift 31).
    """
    z = (seed + n * _GOLDEN) & _M64
    z = ((z ^ (z >> 30)) * _MIX1) & _M64
    z = ((z ^ (z >> 27)) * _MIX2) & _M64
    return z ^ (z >> 31)


def start_vectors(r: int, d_v: int) -> np.ndarray:
    """Deterministic start vectors v0[l] in R^{d_v} for the power method.

    Reading: the top 23 bits m of SplitMix64 output number l*d_v + j + 1 give
    v0[l][j] = (2m + 1 - 2^23) / 2^23, an odd multiple of 2^-23 in (-1, 1),
    exact in fp32 and fp64, identical for every head and every window.
    """
    v0 = np.empty((r, d_v), np.float64)
    for l in range(r):
        for j in range(d_v):
            m = splitmix64(l * d_v + j + 1) >> 41
            v0[l, j] = float((2 * m + 1) - (1 << 23)) / float(1 << 23)
    return v0


# ---------------------------------------------------------------------------
# The exact recurrence [GDN], [KDA]
# ---------------------------------------------------------------------------
def scale_rows(S: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Scale key row i of every head's state by a: a scalar per head [N] (GDN)
    or one factor per key channel [N][d_k] (KDA)."""
    if a.ndim == 1:
        return S * a[:, None, None]
    return S * a[:, :, None]


def exact_step(S, q, k, v, g, beta):
    """One token of the gated delta rule, decay first.

    alpha = exp(g); S' = alpha (.)_rows S; u = beta (v - S'^T k);
    S_t = S' + k u^T; o = S_t^T q. For a scalar alpha this is GDN's
    S_t = alpha (I - beta k k^T) S + beta k v^T; for a per-channel alpha it
    is KDA's S_t = (I - beta k k^T) Diag(alpha) S + beta k v^T.
    Reading: the state that u_t is read from is the decayed one (the only
    reading that is GDN/KDA); the output has no 1/sqrt(d_k) factor.
    Returns (S_t, o_t, u_t).
    """
    Sd = scale_rows(S, np.exp(np.asarray(g, np.float64)))
    beta = np.asarray(beta, np.float64)
    u = beta[:, None] * (v - np.matmul(k[:, None, :], Sd)[:, 0, :])
    Sn = Sd + k[:, :, None] * u[:, None, :]
    o = np.matmul(q[:, None, :], Sn)[:, 0, :]
    return Sn, o, u


# ---------------------------------------------------------------------------
# Window close / encode: compensators, smoothing, quantisation
# [abstract] and [article]: the biggest outliers leave the state as a few
# fp32 rank-one terms with the shape of token updates (the compensator
# tokens); what remains is smoothed per key row and quantised once per window.
# ---------------------------------------------------------------------------
def extract_compensators(S: np.ndarray, r: int, T: int, start: Optional[np.ndarray] = None):
    """E2: r compensators by a fixed-iteration power method with deflation.

    For l = 0..r-1: v <- v0[l]/|v0[l]|; T times: kappa = M v, k = kappa/|kappa|,
    w = M^T k, v = w/|w|. Then comp_k[l] = k (unit key), comp_u[l] = w (the
    least-squares value for that key) and M <- M - k w^T.
    Degenerate head (|kappa|^2 or |w|^2 zero or not finite): compensators
    l..r-1 are zero and M is left as it is.
    start [N][r][d_v] (warm start, not on the pages): where start[n, l] has a
    finite nonzero norm it replaces the fixed start vector v0[l] of head n.
    Returns (comp_k [N][r][d_k], comp_u [N][r][d_v], residual M [N][d_k][d_v]).
    """
    M = np.array(S, dtype=np.float64, copy=True)
    N, dk, dv = M.shape
    ck = np.zeros((N, r, dk))
    cu = np.zeros((N, r, dv))
    live = np.ones(N, bool)
    v0 = start_vectors(r, dv)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        for l in range(r):
            ok = live.copy()
            v = np.repeat((v0[l] / np.sqrt(np.sum(v0[l] ** 2)))[None, :], N, axis=0)
            if start is not None:
                sv = _f64(start[:, l])
                ns = np.sum(sv * sv, axis=1)
                use = np.isfinite(ns) & (ns > 0)
                v = np.where(use[:, None], sv / np.sqrt(np.where(use, ns, 1.0))[:, None], v)
            k = np.zeros((N, dk))
            w = np.zeros((N, dv))
            for _ in range(T):
                kap = np.matmul(M, v[:, :, None])[:, :, 0]
                nk2 = np.sum(kap * kap, axis=1)
                ok &= np.isfinite(nk2) & (nk2 > 0)
                k = np.where(ok[:, None], kap / np.sqrt(np.where(ok, nk2, 1.0))[:, None], 0.0)
                w = np.matmul(k[:, None, :], M)[:, 0, :]
                nw2 = np.sum(w * w, axis=1)
                ok &= np.isfinite(nw2) & (nw2 > 0)
                v = np.where(ok[:, None], w / np.sqrt(np.where(ok, nw2, 1.0))[:, None], 0.0)
            k = np.where(ok[:, None], k, 0.0)
            w = np.where(ok[:, None], w, 0.0)
            ck[:, l] = k
            cu[:, l] = w
            M = M - k[:, :, None] * w[:, None, :]
            live = ok
    return ck, cu, M


def smooth_quantize(R: np.ndarray, bits: int, smoothing: bool = True):
    """E3 + E4 on a residual R [N][d_k][d_v].

    E3 [article, residual smoothing]: s_i = max_j |R_ij| (1 for an all-zero
    row; all ones with smoothing off). E4: Rt = R / s_i; m_j = max_i |Rt_ij|;
    c_j = m_j / Q with Q = 2^(bits-1) - 1; C_ij = clamp(rint(Rt_ij / c_j), -Q, Q)
    rounding half to even, and C = 0 in an all-zero column.
    Returns (s [N][d_k], c [N][d_v], codes int32 [N][d_k][d_v]).
    """
    Q = QMAX[bits]
    R = np.asarray(R, np.float64)
    if smoothing:
        s = np.max(np.abs(R), axis=2)
        s = np.where(s == 0.0, 1.0, s)
    else:
        s = np.ones(R.shape[:2])
    Rt = R / s[:, :, None]
    m = np.max(np.abs(Rt), axis=1)
    c = m / Q
    csafe = np.where(m > 0.0, c, 1.0)
    C = np.where(m[:, None, :] > 0.0, np.clip(np.rint(Rt / csafe[:, None, :]), -Q, Q), 0.0)
    return s, c, C.astype(np.int32)


@dataclass
class Encoded:
    """The low-bit part of a window-start state (one entry per head)."""

    comp_k: np.ndarray   # [N][r][d_k]
    comp_u: np.ndarray   # [N][r][d_v]
    s: np.ndarray        # [N][d_k] key-row smoothing scales
    c: np.ndarray        # [N][d_v] value-column scales
    codes: np.ndarray    # [N][d_k][d_v] int32
    resid: np.ndarray    # [N][d_k][d_v] residual before rounding
    quantized: bool

    def take(self, idx) -> "Encoded":
        resid = None if self.resid is None else self.resid[idx]
        return Encoded(self.comp_k[idx], self.comp_u[idx], self.s[idx], self.c[idx],
                       self.codes[idx], resid, self.quantized)


def encode(S, r: int, T: int, bits: int, smoothing: bool = True, quantize: bool = True,
           start: Optional[np.ndarray] = None) -> Encoded:
    """Enc(S) = E1..E4 (E1: work on a float64 copy of S); start as in
    extract_compensators (warm-started compensators)."""
    ck, cu, R = extract_compensators(S, r, T, start)
    s, c, C = smooth_quantize(R, bits, smoothing)
    return Encoded(ck, cu, s, c, C, R, quantize)


def decode(e: Encoded) -> np.ndarray:
    """Dec = sum_l comp_k[l] comp_u[l]^T + diag(s) C diag(c); with quantisation
    disabled the residual itself replaces diag(s) C diag(c)."""
    lowrank = np.matmul(np.swapaxes(e.comp_k, 1, 2), e.comp_u)
    if not e.quantized:
        return lowrank + e.resid
    return lowrank + e.s[:, :, None] * e.codes.astype(np.float64) * e.c[:, None, :]


# ---------------------------------------------------------------------------
# Plain definition of LeapQuant decoding (the parity reference)
# [abstract], [article]: the state is quantised once at the end of each
# window of W tokens; inside the window the exact recurrence runs.
# ---------------------------------------------------------------------------
def _f64(x):
    return np.asarray(x, np.float64)


@dataclass
class CloseEvent:
    step: int
    heads: np.ndarray          # indices of the heads that closed
    folded: np.ndarray         # dense state before Enc, [n][d_k][d_v]
    enc: Encoded


def run_dense(S_init, tokens: Iterable[Dict[str, np.ndarray]], win_len, win_off, *, r: int,
              T: int = 4, bits: int = 8, smoothing: bool = True, quantize: bool = True,
              record: bool = False, rounding_noise: float = 0.0, noise_seed: int = 0,
              warm_start: bool = False):
    """Run LeapQuant decoding as its plain definition.

    S <- Dec(Enc(S_init)); for each token: S <- exact step; when the head's
    window ends with this token, S <- Dec(Enc(S)).
    Readings: the close comes after the W-th token's update and output (so
    o_W uses the unquantised state); window position starts at the head's
    offset with nothing buffered; every head of a sequence shares its window.

    rounding_noise > 0 is not part of the method: every state entering Enc is
    first multiplied entrywise by (1 + rounding_noise * N(0,1)). With a noise
    of fp32 rounding size this measures how well the plain definition's
    outputs are determined by its inputs (rounding decisions near ties).

    warm_start (a variant, not on the pages): each close starts compensator l's
    power method from the same head's compensator value u_l of the window
    that is closing (the fixed start vector where that is zero); the initial
    encode starts cold.

    S_init [N][d_k][d_v]; tokens yields per-step dicts with q, k [N][d_k],
    v [N][d_v], g [N] or [N][d_k], beta [N]; win_len, win_off [N].
    Returns dict(o [T][N][d_v], u [T][N][d_v], S final, enc0, closes).
    """
    rng = np.random.default_rng(noise_seed)

    def enc(X, start=None):
        if rounding_noise:
            X = X * (1.0 + rounding_noise * rng.standard_normal(X.shape))
        return encode(X, r, T, bits, smoothing, quantize, start)

    enc0 = enc(_f64(S_init))
    comp_u = enc0.comp_u.copy()
    S = decode(enc0)
    pos = np.array(win_off, np.int64).copy()
    W = np.array(win_len, np.int64)
    outs, us, closes = [], [], []
    for t, tok in enumerate(tokens):
        S, o, u = exact_step(S, _f64(tok["q"]), _f64(tok["k"]), _f64(tok["v"]), tok["g"], tok["beta"])
        outs.append(o)
        us.append(u)
        pos += 1
        idx = np.nonzero(pos == W)[0]
        if idx.size:
            e = enc(S[idx], comp_u[idx] if warm_start else None)
            if record:
                closes.append(CloseEvent(t, idx, S[idx].copy(), e))
            S[idx] = decode(e)
            comp_u[idx] = e.comp_u
            pos[idx] = 0
    return dict(o=np.array(outs), u=np.array(us), S=S, enc0=enc0, closes=closes)


# ---------------------------------------------------------------------------
# Buffered form: what a decode kernel computes inside a window, written
# separately from run_dense. Used to pin the window algebra.
# [abstract]: within a window an output reads the frozen quantised state and
# the fp32 updates buffered so far; compensators are handled exactly like
# buffered token updates (they sit at window position 0 and decay with the
# residual).
# ---------------------------------------------------------------------------
class BufferedOracle:
    """State = (window-start Enc, buffer of (k_m, u_m, G_m)), G = cumulative
    log-decay since the window start (scalar per head for GDN, per key channel
    for KDA)."""

    def __init__(self, S_init, win_len, win_off, *, w_max: int, r: int, T: int = 4,
                 bits: int = 8, smoothing: bool = True, quantize: bool = True, kda: bool = False,
                 warm_start: bool = False):
        S_init = _f64(S_init)
        self.N, self.dk, self.dv = S_init.shape
        self.r, self.T, self.bits, self.smoothing, self.quantize, self.kda = r, T, bits, smoothing, quantize, kda
        self.warm_start = warm_start
        self.w_max = w_max
        self.W = np.array(win_len, np.int64)
        self.pos = np.array(win_off, np.int64).copy()
        self.base = encode(S_init, r, T, bits, smoothing, quantize)
        N, dk, dv = self.N, self.dk, self.dv
        self.buf_k = np.zeros((N, w_max, dk))
        self.buf_u = np.zeros((N, w_max, dv))
        self.buf_G = np.zeros((N, w_max, dk) if kda else (N, w_max))
        self.n = np.zeros(N, np.int64)
        self.closes: List[CloseEvent] = []

    def _G_now(self):
        """Cumulative log-decay of the last buffered token (0 on an empty buffer)."""
        ar = np.arange(self.N)
        last = self.buf_G[ar, np.maximum(self.n - 1, 0)]
        empty = self.n == 0
        if self.kda:
            return np.where(empty[:, None], 0.0, last)
        return np.where(empty, 0.0, last)

    def _base_readout(self, xbar):
        """Window-start state read against x: Dec(...)^T xbar, kept in factored form."""
        b = self.base
        kap = np.einsum("nli,ni->nl", b.comp_k, xbar)
        y = np.einsum("nlj,nl->nj", b.comp_u, kap)
        if b.quantized:
            y = y + b.c * np.einsum("nij,ni->nj", b.codes.astype(np.float64), b.s * xbar)
        else:
            y = y + np.einsum("nij,ni->nj", b.resid, xbar)
        return y

    def _buffer_readout(self, G, x):
        """sum_m u_m (k_m . (exp(G - G_m) (.) x)) over the buffered entries."""
        valid = np.arange(self.w_max)[None, :] < self.n[:, None]          # [N][W]
        if self.kda:
            rho = np.exp(G[:, None, :] - self.buf_G) * valid[:, :, None]    # [N][W][d_k]
            kap = np.einsum("nmi,nmi,ni->nm", self.buf_k, rho, x)
        else:
            rho = np.exp(G[:, None] - self.buf_G) * valid                   # [N][W]
            kap = rho * np.einsum("nmi,ni->nm", self.buf_k, x)
        return np.einsum("nmj,nm->nj", self.buf_u, kap)

    def step(self, q, k, v, g, beta):
        q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
        if np.any(self.n >= self.w_max):
            raise ValueError("window buffer full: close before the next token")
        G = self._G_now() + g
        eG = np.exp(G)
        ys = []
        for x in (k, q):
            xbar = (eG[:, None] * x) if not self.kda else eG * x
            ys.append(self._base_readout(xbar) + self._buffer_readout(G, x))
        yk, yq = ys
        u = beta[:, None] * (v - yk)
        o = yq + np.sum(k * q, axis=1)[:, None] * u
        ar = np.arange(self.N)
        self.buf_k[ar, self.n] = k
        self.buf_u[ar, self.n] = u
        self.buf_G[ar, self.n] = G
        self.n += 1
        self.pos += 1
        return o, u

    def fold(self, idx) -> np.ndarray:
        """Dense state of heads idx: exp(G_n) (.)_rows S0 + sum_m exp(G_n - G_m) (.)_rows k_m u_m^T."""
        G = self._G_now()[idx]
        S0 = decode(self.base.take(idx))
        n = self.n[idx]
        valid = np.arange(self.w_max)[None, :] < n[:, None]
        if self.kda:
            S = np.exp(G)[:, :, None] * S0
            rho = np.exp(G[:, None, :] - self.buf_G[idx]) * valid[:, :, None]
            S = S + np.einsum("nmi,nmi,nmj->nij", rho, self.buf_k[idx], self.buf_u[idx])
        else:
            S = np.exp(G)[:, None, None] * S0
            rho = np.exp(G[:, None] - self.buf_G[idx]) * valid
            S = S + np.einsum("nm,nmi,nmj->nij", rho, self.buf_k[idx], self.buf_u[idx])
        return S

    def close_due(self, t: int = -1):
        """Close every head whose window ended: fold, re-encode, empty the buffer."""
        idx = np.nonzero(self.pos == self.W)[0]
        if idx.size == 0:
            return idx
        S = self.fold(idx)
        start = self.base.comp_u[idx] if self.warm_start else None
        e = encode(S, self.r, self.T, self.bits, self.smoothing, self.quantize, start)
        self.closes.append(CloseEvent(t, idx, S, e))
        for name in ("comp_k", "comp_u", "s", "c", "codes", "resid"):
            getattr(self.base, name)[idx] = getattr(e, name)
        self.n[idx] = 0
        self.pos[idx] = 0
        return idx


def run_buffered(S_init, tokens, win_len, win_off, *, w_max: int, r: int, T: int = 4, bits: int = 8,
                 smoothing: bool = True, quantize: bool = True, kda: bool = False, warm_start: bool = False):
    st = BufferedOracle(S_init, win_len, win_off, w_max=w_max, r=r, T=T, bits=bits,
                        smoothing=smoothing, quantize=quantize, kda=kda, warm_start=warm_start)
    outs, us = [], []
    for t, tok in enumerate(tokens):
        o, u = st.step(tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"])
        outs.append(o)
        us.append(u)
        st.close_due(t)
    return dict(o=np.array(outs), u=np.array(us), state=st)


# ---------------------------------------------------------------------------
# Naive per-token requantisation, written element by element (small sizes
# only). With no compensators and a window of one token LeapQuant must reduce
# to this; with smoothing off it is the plain INT8 state of [article].
# ---------------------------------------------------------------------------
def run_per_token(S_init, tokens, *, bits: int = 8, smoothing: bool = True):
    Q = QMAX[bits]

    def requant(S):
        N, dk, dv = S.shape
        out = np.zeros_like(S)
        for n in range(N):
            s = [1.0] * dk
            if smoothing:
                for i in range(dk):
                    mx = max(abs(S[n, i, j]) for j in range(dv))
                    s[i] = mx if mx != 0.0 else 1.0
            for j in range(dv):
                col = [S[n, i, j] / s[i] for i in range(dk)]
                m = max(abs(x) for x in col)
                if m == 0.0:
                    continue
                cj = m / Q
                for i in range(dk):
                    code = min(max(float(np.rint(col[i] / cj)), -Q), Q)
                    out[n, i, j] = s[i] * code * cj
        return out

    S = requant(_f64(S_init))
    outs = []
    for tok in tokens:
        q, k, v, g, beta = (_f64(tok[x]) for x in ("q", "k", "v", "g", "beta"))
        N, dk, dv = S.shape
        o = np.zeros((N, dv))
        for n in range(N):
            a = np.exp(g[n])
            for i in range(dk):
                S[n, i, :] *= (a if np.ndim(a) == 0 else a[i])
            for j in range(dv):
                pred = sum(S[n, i, j] * k[n, i] for i in range(dk))
                uj = beta[n] * (v[n, j] - pred)
                for i in range(dk):
                    S[n, i, j] += k[n, i] * uj
            for j in range(dv):
                o[n, j] = sum(S[n, i, j] * q[n, i] for i in range(dk))
        outs.append(o)
        S = requant(S)
    return dict(o=np.array(outs), S=S)


# ---------------------------------------------------------------------------
# Helpers the parity protocol needs
# ---------------------------------------------------------------------------
def fold_window(S0, buf_k, buf_u, buf_G, n, kda: bool) -> np.ndarray:
    """Dense state after n buffered tokens from window-start state S0.

    S0 [N][d_k][d_v]; buf_k [N][W][d_k]; buf_u [N][W][d_v];
    buf_G [N][W] (GDN) or [N][W][d_k] (KDA); n [N].
    """
    S0, buf_k, buf_u, buf_G = _f64(S0), _f64(buf_k), _f64(buf_u), _f64(buf_G)
    N, W = buf_k.shape[:2]
    n = np.asarray(n, np.int64)
    valid = np.arange(W)[None, :] < n[:, None]
    last = np.maximum(n - 1, 0)
    Gn = buf_G[np.arange(N), last]
    if kda:
        Gn = np.where((n == 0)[:, None], 0.0, Gn)
        rho = np.exp(Gn[:, None, :] - buf_G) * valid[:, :, None]
        return np.exp(Gn)[:, :, None] * S0 + np.einsum("nmi,nmi,nmj->nij", rho, buf_k, buf_u)
    Gn = np.where(n == 0, 0.0, Gn)
    rho = np.exp(Gn[:, None] - buf_G) * valid
    return np.exp(Gn)[:, None, None] * S0 + np.einsum("nm,nmi,nmj->nij", rho, buf_k, buf_u)


# ---------------------------------------------------------------------------
# Prefill handoff. [article] and [abstract] quantize the recurrent state once
# per window of decoded tokens; the prompt before decoding runs at full
# precision (reading: the exact recurrence) and its final state enters the
# LeapQuant form once, by the encode above, as a window start with an empty
# buffer.
# ---------------------------------------------------------------------------
def prefill(S_init, tokens: Iterable[Dict[str, np.ndarray]]):
    """The exact gated delta rule over the prompt tokens in order; returns
    (S after the prompt, [o_t for every prompt token])."""
    S = _f64(S_init)
    outs: List[np.ndarray] = []
    for tk in tokens:
        S, o, _ = exact_step(S, _f64(tk["q"]), _f64(tk["k"]), _f64(tk["v"]), tk["g"], tk["beta"])
        outs.append(o)
    return S, outs


def prefill_handoff(S_init, tokens, *, r: int, T: int = 4, bits: int = 8, smoothing: bool = True):
    """prefill(), then the encode of its final state: the window-start state
    decoding continues from. Returns (Encoded, S after the prompt, outputs)."""
    S, outs = prefill(S_init, tokens)
    return encode(S, r, T, bits, smoothing), S, outs


def outlier_ratio(X: np.ndarray) -> np.ndarray:
    """max |X| / median |X| per head (the pages' outlier-to-median measure,
    [article] residual-smoothing paragraph; the exact statistic is a reading)."""
    A = np.abs(_f64(X)).reshape(X.shape[0], -1)
    return A.max(axis=1) / np.median(A, axis=1)

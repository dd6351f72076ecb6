"""Small seeded inputs for the oracle pins (no method arithmetic here)."""
import numpy as np


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_tokens(rng, steps, N, dk, dv, kda=False, decay_scale=0.05, beta=None):
    toks = []
    for _ in range(steps):
        g = -np.logaddexp(0.0, rng.standard_normal((N, dk) if kda else N)) * decay_scale
        toks.append(dict(
            q=unit(rng.standard_normal((N, dk))),
            k=unit(rng.standard_normal((N, dk))),
            v=rng.standard_normal((N, dv)),
            g=g,
            beta=(1.0 / (1.0 + np.exp(-rng.standard_normal(N)))) if beta is None else np.full(N, float(beta)),
        ))
    return toks


def planted_state(rng, N, dk, dv, sigma=0.1, rows=2, rmul=50.0, cols=1, cmul=20.0):
    S = rng.normal(0.0, sigma, (N, dk, dv))
    for n in range(N):
        S[n, rng.choice(dk, rows, replace=False), :] *= rmul
        S[n, :, rng.choice(dv, cols, replace=False)] *= cmul
    return S


def flat_steps(tok):
    """Token chunk [n][S][H][...] from the workload stream -> per-step dicts over
    N = S*H heads, float64."""
    n = tok["q"].shape[0]
    out = []
    for t in range(n):
        d = {}
        for key in ("q", "k", "v", "g", "beta"):
            a = tok[key][t]
            d[key] = a.reshape((-1,) + a.shape[2:]).astype(np.float64)
        out.append(d)
    return out


def rel_l2(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))

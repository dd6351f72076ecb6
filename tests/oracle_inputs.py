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

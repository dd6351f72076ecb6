"""Seeded workload generators: determinism, chunking, shapes, distributions."""
import numpy as np
import pytest

from linear_attention_recurrent_kda_amd import workloads as wk


def test_workload_shapes():
    w = wk.WORKLOADS
    assert (w["tiny_gdn"].batch, w["tiny_gdn"].heads, w["tiny_gdn"].d_k) == (1, 1, 32)
    assert (w["qwen_gdn"].batch, w["qwen_gdn"].heads, w["qwen_gdn"].d_k, w["qwen_gdn"].n_comp) == (64, 32, 128, 4)
    assert w["kda_int4"].bits == 4 and w["kda_int4"].kda
    assert w["prefix_mix"].w_max == 32 and w["prefix_mix"].staggered


def test_chunked_draws_equal_one_draw():
    wl = wk.WORKLOADS["qwen_gdn"].replace(batch=3, heads=2)
    a = wk.TokenStream(wl, [0, 2]).next(10)
    s = wk.TokenStream(wl, [0, 2])
    b1, b2 = s.next(4), s.next(6)
    for key in a:
        assert np.array_equal(a[key], np.concatenate([b1[key], b2[key]]))
    # a subset regenerates the same values as the full batch
    full = wk.TokenStream(wl).next(10)
    assert np.array_equal(full["q"][:, [0, 2]], a["q"])


def test_token_distributions():
    wl = wk.WORKLOADS["tiny_gdn"]
    t = wk.TokenStream(wl).next(64)
    assert np.allclose(np.linalg.norm(t["q"], axis=-1), 1.0, atol=1e-6)
    assert np.allclose(np.linalg.norm(t["k"], axis=-1), 1.0, atol=1e-6)
    assert np.all((t["beta"] > 0) & (t["beta"] < 1))
    assert np.all(t["g"] < 0) and np.all(t["g"] > -1.0)


def test_bf16_rounding_and_uniform_decay():
    wl = wk.WORKLOADS["qwen_gdn"].replace(batch=2, heads=3)
    t = wk.TokenStream(wl).next(5)
    assert np.array_equal(wk.bf16_to_f32(t["q16"]), t["q"])
    assert np.allclose(np.linalg.norm(t["k"], axis=-1), 1.0, atol=1e-2)
    alpha = np.exp(t["g"].astype(np.float64))
    assert np.all((alpha >= 0.9 - 1e-6) & (alpha < 1.0))
    # round to nearest even on a few hand-made bit patterns
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], np.float32)
    assert list(wk.round_to_bf16(x)) == [0x3F80, 0x3F80, 0x3F82, 0xC020]


def test_planted_outliers_and_kda_decay():
    wl = wk.WORKLOADS["kda_int4"].replace(batch=2, heads=4)
    S = wk.initial_states(wl, [0, 1])
    assert S.shape == (2, 4, 128, 128) and S.dtype == np.float32
    row_norm = np.linalg.norm(S, axis=3)
    assert np.all(np.sort(row_norm, axis=2)[:, :, -2:] > 10 * np.median(row_norm, axis=2)[..., None])
    lam = wk.kda_lambda(wl)
    assert lam.shape == (4, 128) and lam.min() >= 0.01 and lam.max() <= 0.2
    t = wk.TokenStream(wl).next(3)
    assert t["g"].shape == (3, 2, 4, 128) and np.all(t["g"] < 0)


def test_window_schedule():
    wl = wk.WORKLOADS["prefix_mix"].replace(batch=8)
    W, off = wk.window_lengths(wl), wk.window_offsets(wl)
    assert list(W) == [16, 32] * 4
    assert np.all((off >= 0) & (off < 16)) and len(set(off.tolist())) > 1
    assert np.all(wk.window_offsets(wk.WORKLOADS["qwen_gdn"]) == 0)

"""C ABI host tests (CPU only): the library loads and exports every function
include/leapquant.h declares; argument validation returns the documented codes
before anything reaches the GPU; the host helpers compute sizes and close
lists. No call here passes validation, so no kernel is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

from linear_attention_recurrent_kda_amd import leapquant as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "leapquant.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert set(names) == set(L.EXPORTS), names
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def dims(**kw):
    base = dict(batch=2, heads=3, d_k=128, d_v=128, w_max=16, n_comp=4, bits=8, decay_per_channel=0,
                act_dtype=0, smoothing=1, power_iters=4, warm_start=0)
    base.update(kw)
    return L.CDims(**base)


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def state(**kw):
    p = {n: FAKE + 0x1000 * i for i, n in enumerate(L.STATE_FIELDS)}
    p.update(kw)
    return L.CState(**p)


def step(d, st, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE):
    return L.raw_call("leapquant_decode_step", ctypes.byref(d), ctypes.byref(st), q, k, v, g, beta, o, None)


@pytest.mark.parametrize("kw,code", [
    (dict(d_k=96, d_v=96), L.LQ_ERR_SHAPE),
    (dict(d_k=128, d_v=64), L.LQ_ERR_SHAPE),
    (dict(batch=-1), L.LQ_ERR_SHAPE),
    (dict(bits=5), L.LQ_ERR_BITS),
    (dict(bits=7), L.LQ_ERR_BITS),
    (dict(w_max=0), L.LQ_ERR_CONFIG),
    (dict(w_max=65), L.LQ_ERR_CONFIG),
    (dict(n_comp=9), L.LQ_ERR_CONFIG),
    (dict(power_iters=0), L.LQ_ERR_CONFIG),
    (dict(act_dtype=2), L.LQ_ERR_CONFIG),
    (dict(decay_per_channel=2), L.LQ_ERR_CONFIG),
    (dict(smoothing=3), L.LQ_ERR_CONFIG),
    (dict(warm_start=2), L.LQ_ERR_CONFIG),
])
def test_dims_validation(kw, code):
    d = dims(**kw)
    st = state()
    assert step(d, st) == code
    if "w_max" not in kw:
        assert step_at(d, st, 3) == code
    assert L.raw_call("leapquant_window_close", ctypes.byref(d), ctypes.byref(st), None, 0, None, None) == code
    assert L.raw_call("leapquant_encode", ctypes.byref(d), FAKE, ctypes.byref(st), None, None) == code
    sizes = (ctypes.c_size_t * L.LQ_STATE_NBUF)()
    assert L.raw_call("lq_state_sizes", ctypes.byref(d), sizes) == code


def step_at(d, st, n, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE):
    return L.raw_call("leapquant_decode_step_at", ctypes.byref(d), ctypes.byref(st), n, q, k, v, g, beta, o, None)


def test_decode_step_at_validation():
    """The position must lie in [0, w_max); the other arguments are checked as
    for leapquant_decode_step."""
    d = dims()
    assert step_at(d, state(), -1) == L.LQ_ERR_CONFIG
    assert step_at(d, state(), 16) == L.LQ_ERR_CONFIG
    assert step_at(dims(w_max=32), state(), 40) == L.LQ_ERR_CONFIG
    assert step_at(d, state(codes=None), 0) == L.LQ_ERR_NULL
    assert step_at(d, state(), 15, q=None) == L.LQ_ERR_NULL
    assert step_at(d, state(ent_g=FAKE + 8), 2) == L.LQ_ERR_ALIGN
    assert step_at(d, state(), 2, o=FAKE + 4) == L.LQ_ERR_ALIGN


def decode_close_at(d, st, n, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE, dbg=None):
    return L.raw_call("leapquant_decode_close_at", ctypes.byref(d), ctypes.byref(st), n, q, k, v, g, beta, o,
                      dbg, None)


def test_decode_close_at_validation():
    """The window's last token plus its close: the position must lie in
    [0, w_max); activations, outputs, state and the optional residual are
    checked as for leapquant_decode_step and leapquant_window_close."""
    d = dims()
    assert decode_close_at(d, state(), -1) == L.LQ_ERR_CONFIG
    assert decode_close_at(d, state(), 16) == L.LQ_ERR_CONFIG
    assert decode_close_at(dims(bits=5), state(), 15) == L.LQ_ERR_BITS
    assert decode_close_at(dims(power_iters=0), state(), 15) == L.LQ_ERR_CONFIG
    assert decode_close_at(d, state(buf_len=None), 15) == L.LQ_ERR_NULL
    assert decode_close_at(d, state(), 15, beta=None) == L.LQ_ERR_NULL
    assert decode_close_at(d, state(), 15, o=FAKE + 4) == L.LQ_ERR_ALIGN
    assert decode_close_at(d, state(), 15, dbg=FAKE + 4) == L.LQ_ERR_ALIGN
    assert decode_close_at(d, state(ent_u=FAKE + 4), 15) == L.LQ_ERR_ALIGN
    assert decode_close_at(dims(batch=0), state(), 15) == L.LQ_OK   # nothing to do, nothing launched


def test_null_and_alignment_validation():
    d = dims()
    assert L.raw_call("leapquant_decode_step", None, None, None, None, None, None, None, None, None) == L.LQ_ERR_NULL
    assert step(d, state(codes=None)) == L.LQ_ERR_NULL
    for f in ("ent_k", "ent_u", "ent_g", "buf_len", "row_scale"):
        assert step(d, state(**{f: None})) == L.LQ_ERR_NULL, f
    assert step(d, state(), q=None) == L.LQ_ERR_NULL
    assert step(d, state(codes=FAKE + 4)) == L.LQ_ERR_ALIGN
    assert step(d, state(ent_g=FAKE + 8)) == L.LQ_ERR_ALIGN
    assert step(d, state(ent_u=FAKE + 4)) == L.LQ_ERR_ALIGN
    assert step(d, state(err=FAKE + 2)) == L.LQ_ERR_ALIGN
    assert step(d, state(), q=FAKE + 2) == L.LQ_ERR_ALIGN
    assert step(d, state(), v=FAKE + 8) == L.LQ_ERR_ALIGN   # fp32 rows move in 16-byte pieces
    assert step(d, state(), o=FAKE + 4) == L.LQ_ERR_ALIGN
    assert step(d, state(), g=FAKE + 2) == L.LQ_ERR_ALIGN
    db = dims(act_dtype=1)
    assert step(db, state(), q=FAKE + 1) == L.LQ_ERR_ALIGN
    assert step(db, state(), v=FAKE + 4) == L.LQ_ERR_ALIGN  # bf16 rows move in 8-byte pieces
    # r == 0: the entry arrays hold only the token buffer, still required and aligned
    assert step(dims(n_comp=0), state(ent_k=None)) == L.LQ_ERR_NULL
    assert step(dims(n_comp=0), state(ent_u=FAKE + 4)) == L.LQ_ERR_ALIGN
    assert L.raw_call("gdn_decode_fp32_baseline", ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                      None) == L.LQ_ERR_NULL
    assert L.raw_call("gdn_decode_fp32_baseline", ctypes.byref(d), FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE,
                      FAKE, None) == L.LQ_ERR_ALIGN
    assert L.raw_call("leapquant_encode", ctypes.byref(d), None, ctypes.byref(state()), None, None) == L.LQ_ERR_NULL
    assert L.raw_call("leapquant_encode", ctypes.byref(d), FAKE, ctypes.byref(state()), FAKE + 4,
                      None) == L.LQ_ERR_ALIGN
    assert L.raw_call("leapquant_dequantize", ctypes.byref(d), ctypes.byref(state()), None, None) == L.LQ_ERR_NULL


def test_prefill_validation():
    d = dims()
    pf = lambda S, n, q=FAKE, st=None: L.raw_call("leapquant_prefill", ctypes.byref(d), S, n, q, FAKE, FAKE, FAKE,
                                                  FAKE, FAKE, st, None)
    assert pf(FAKE, -1) == L.LQ_ERR_CONFIG
    assert pf(None, 4) == L.LQ_ERR_NULL
    assert pf(FAKE + 4, 4) == L.LQ_ERR_ALIGN
    assert pf(FAKE, 4, q=None) == L.LQ_ERR_NULL
    assert pf(FAKE, 4, q=FAKE + 2) == L.LQ_ERR_ALIGN
    assert pf(FAKE, 0, st=ctypes.byref(state(codes=None))) == L.LQ_ERR_NULL
    bad = dims(bits=5)
    assert L.raw_call("leapquant_prefill", ctypes.byref(bad), FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                      ctypes.byref(state()), None) == L.LQ_ERR_BITS
    e = dims(batch=0)
    assert L.raw_call("leapquant_prefill", ctypes.byref(e), None, 4, None, None, None, None, None, None, None,
                      None) == L.LQ_OK


def test_snapshot_sizes_and_validation():
    assert L.snapshot_bytes(L.Dims(64, 32, 128, n_comp=4, bits=8)) == 128 * 128 + 8 * 128 + 8 * 4 * 128
    assert L.snapshot_bytes(L.Dims(64, 32, 128, n_comp=4, bits=4)) == 128 * 64 + 8 * 128 + 8 * 4 * 128
    assert L.snapshot_bytes(L.Dims(1, 1, 32, n_comp=2, bits=6)) == 32 * 24 + 8 * 32 + 8 * 2 * 32
    d = dims()
    for fn in ("leapquant_snapshot", "leapquant_restore"):
        call = lambda st, ids, n, snap: L.raw_call(fn, ctypes.byref(d), ctypes.byref(st), ids, n, snap, None)
        assert call(state(), None, 0, None) == L.LQ_ERR_NULL
        assert call(state(), None, 0, FAKE + 4) == L.LQ_ERR_ALIGN
        assert call(state(), FAKE, 3, FAKE) == L.LQ_ERR_CONFIG
        assert call(state(), FAKE, 0, None) == L.LQ_OK          # empty list: nothing to do
        assert call(state(ent_k=None), None, 0, FAKE) == L.LQ_ERR_NULL
        assert L.raw_call(fn, ctypes.byref(dims(bits=5)), ctypes.byref(state()), None, 0, FAKE, None) == L.LQ_ERR_BITS


def test_close_list_argument_validation():
    d = dims()
    st = state()
    close = lambda ids, n: L.raw_call("leapquant_window_close", ctypes.byref(d), ctypes.byref(st), ids, n,
                                      None, None)
    assert close(FAKE, 3) == L.LQ_ERR_CONFIG       # more ids than sequences
    assert close(FAKE, -1) == L.LQ_ERR_CONFIG
    assert close(FAKE, 0) == L.LQ_OK               # empty list: nothing to do
    assert close(FAKE + 2, 1) == L.LQ_ERR_ALIGN


def test_empty_batch_is_a_no_op():
    for kw in (dict(batch=0), dict(heads=0)):
        d = dims(**kw)
        empty = L.CState()
        assert step(d, empty, None, None, None, None, None, None) == L.LQ_OK
        assert L.raw_call("leapquant_encode", ctypes.byref(d), None, ctypes.byref(empty), None, None) == L.LQ_OK
        assert L.raw_call("leapquant_window_close", ctypes.byref(d), ctypes.byref(empty), None, 0, None,
                          None) == L.LQ_OK
        assert L.raw_call("gdn_decode_fp32_baseline", ctypes.byref(d), None, None, None, None, None, None, None,
                          None) == L.LQ_OK


def test_state_sizes():
    s = L.state_sizes(L.Dims(64, 32, 128, w_max=16, n_comp=4, bits=8))
    BH = 64 * 32
    assert s["codes"] == BH * 128 * 128 and s["ent_g"] == BH * (4 + 16) * 4 and s["err"] == 4
    assert s["ent_k"] == s["ent_u"] == BH * (4 + 16) * 128 * 4
    assert s["row_scale"] == s["col_scale"] == BH * 128 * 4 and s["buf_len"] == BH * 4
    s4 = L.state_sizes(L.Dims(128, 32, 128, w_max=16, n_comp=4, bits=4, kda=True))
    assert s4["codes"] == 128 * 32 * 128 * 64 and s4["ent_g"] == 128 * 32 * (4 + 16) * 128 * 4
    s6 = L.state_sizes(L.Dims(64, 32, 128, w_max=16, n_comp=4, bits=6))
    assert s6["codes"] == BH * 128 * 96  # 6-bit: two planes, 96 bytes per value column
    s0 = L.state_sizes(L.Dims(2, 3, 32, w_max=1, n_comp=0))
    assert s0["ent_k"] == 6 * 1 * 32 * 4


def test_close_list_matches_schedule():
    rng = np.random.default_rng(0)
    W = np.where(np.arange(40) % 2 == 0, 16, 32).astype(np.int32)
    off = rng.integers(0, 16, 40).astype(np.int32)
    for t in range(70):
        want = [b for b in range(40) if (off[b] + t + 1) % W[b] == 0]
        assert list(L.close_list(W, off, t)) == want
    with pytest.raises(L.LeapQuantError):
        L.close_list(np.array([16], np.int32), np.array([16], np.int32), 0)  # offset outside the window
    with pytest.raises(L.LeapQuantError):
        L.close_list(np.array([0], np.int32), np.array([0], np.int32), 0)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.status_string(code) != "unknown status"
    assert L.status_string(-99) == "unknown status"


def test_buffered_tokens_follow_the_close_schedule():
    """runner.buffered_tokens (the position handed to leapquant_decode_step_at)
    against a token-by-token count: every sequence starts empty, gains one
    token per step and empties after each close of its list."""
    from linear_attention_recurrent_kda_amd import runner

    rng = np.random.default_rng(1)
    W = np.where(np.arange(24) % 3 == 0, 16, 32).astype(np.int32)
    off = rng.integers(0, 16, 24).astype(np.int32)
    n = np.zeros(24, np.int64)
    for t in range(100):
        assert np.array_equal(runner.buffered_tokens(W, off, t), n), t
        n += 1
        n[L.close_list(W, off, t)] = 0
    # aligned windows: every sequence at the same position, t mod W
    W16, zero = np.full(8, 16, np.int32), np.zeros(8, np.int32)
    assert [int(runner.buffered_tokens(W16, zero, t)[0]) for t in range(40)] == [t % 16 for t in range(40)]

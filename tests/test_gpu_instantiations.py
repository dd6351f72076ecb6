"""Every kernel instantiation the C ABI can dispatch, against the fp64 oracle.

The decode step, the window close / encode and the FP32 baseline are compiled
for d in {32, 64, 128}, 8-, 6- and 4-bit codes, scalar (GDN) and per-channel
(KDA) decay, fp32 and bf16 activations. Each instantiation here gets the
check of its row on a small batch:
  decode step: G4, one token from an oracle-made state uploaded in fp32,
     o_t and u_t <= 1e-5 relative, at a buffer length inside the 24 entries
     whose rows are prefetched and at one past them (r + n > 24), so both
     entry paths run;
  close and encode: G1 (codes >= 99.99% identical to the oracle's
     quantization of the GPU's own residual, all within one LSB, row scales
     bit-identical, column scales within 2 ulp) and G2 (compensators plus
     residual rebuild the oracle's fold of the GPU's pre-close buffers, or the
     dense input, to <= 1e-6), with 21 buffered tokens (two fold passes of
     16 entries, the second ragged);
  FP32 baseline: 8 exact tokens against the oracle's exact recurrence, o and
     the final state <= 1e-5 relative.
"""
import itertools

import numpy as np
import pytest
import torch

from linear_attention_recurrent_kda_amd import leapquant as lqk
from linear_attention_recurrent_kda_amd import runner
from linear_attention_recurrent_kda_amd import workloads as wk
from oracle import leapquant_oracle as lq
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

DIMS = (32, 64, 128)
BITS = (8, 6, 4)


def _wl(d, kda, bf16, window=32, r=4, batch=2, heads=2):
    return wk.WORKLOADS["tiny_gdn"].replace(batch=batch, heads=heads, d_k=d, d_v=d, kda=kda, act_bf16=bf16,
                                            window=window, n_comp=r, steps=64)


@pytest.mark.parametrize("d,bits,kda,bf16,n_pre", [
    (d, b, k, f, n) for d, b, k, f in itertools.product(DIMS, BITS, (False, True), (False, True)) for n in (3, 26)])
def test_decode_step_every_instantiation(d, bits, kda, bf16, n_pre):
    wl = _wl(d, kda, bf16)
    seqs = list(range(wl.batch))
    N = wl.batch * wl.heads
    dims = runner.dims_for(wl, bits)
    assert wl.n_comp + n_pre + 1 <= wl.n_comp + dims.w_max
    S0 = wk.initial_states(wl, seqs).reshape(-1, d, d).astype(np.float64)
    toks = gh.flat_steps(wk.TokenStream(wl, seqs).next(n_pre + 1))
    bo = lq.BufferedOracle(S0, np.full(N, 10 ** 6), np.zeros(N), w_max=dims.w_max, r=wl.n_comp,
                           T=wl.power_iters, bits=bits, smoothing=wl.smoothing, kda=kda)
    for t in toks[:n_pre]:
        bo.step(t["q"], t["k"], t["v"], t["g"], t["beta"])
    r32 = lambda x: np.asarray(x, np.float32).astype(np.float64)
    for f in ("comp_k", "comp_u", "s", "c"):
        setattr(bo.base, f, r32(getattr(bo.base, f)))
    bo.buf_k, bo.buf_u, bo.buf_G = r32(bo.buf_k), r32(bo.buf_u), r32(bo.buf_G)
    st = lqk.State(dims)
    gh.upload_state(st, dims, bo.base, bo.buf_k, bo.buf_u, bo.buf_G, bo.n)
    last = toks[n_pre]
    o_ref, u_ref = bo.step(last["q"], last["k"], last["v"], last["g"], last["beta"])
    raw = wk.TokenStream(wl, seqs).next(n_pre + 1)
    dev = runner.upload_tokens({k: v[n_pre:] for k, v in raw.items()}, bf16)
    o = torch.empty((N, d), dtype=torch.float32, device="cuda")
    lqk.decode_step(dims, st, dev["q"][0], dev["k"][0], dev["v"][0], dev["g"][0], dev["beta"][0], o)
    host = gh.download_state(st, dims)
    u_gpu = host["buf_u"][np.arange(N), n_pre]
    eo, eu = gh.rel_l2(o.cpu().numpy(), o_ref), gh.rel_l2(u_gpu, u_ref)
    print(d, bits, kda, bf16, n_pre, eo, eu)
    assert eo <= 1e-5 and eu <= 1e-5
    assert int(st.err.item()) == 0
    assert np.all(host["buf_len"] == n_pre + 1)
    assert np.array_equal(host["buf_k"][np.arange(N), n_pre], np.asarray(last["k"], np.float32))
    if kda:
        G_ref = np.asarray(bo.buf_G[np.arange(N), n_pre], np.float32)
        np.testing.assert_allclose(host["buf_g"][np.arange(N), n_pre], G_ref, rtol=1e-6, atol=1e-7)


def _uploaded_pair(d, bits, kda, bf16, n_pre):
    """Two device states holding the same oracle-made state with n_pre buffered
    tokens, and the next token's device inputs."""
    wl = _wl(d, kda, bf16)
    seqs = list(range(wl.batch))
    N = wl.batch * wl.heads
    dims = runner.dims_for(wl, bits)
    S0 = wk.initial_states(wl, seqs).reshape(-1, d, d).astype(np.float64)
    bo = lq.BufferedOracle(S0, np.full(N, 10 ** 6), np.zeros(N), w_max=dims.w_max, r=wl.n_comp,
                           T=wl.power_iters, bits=bits, smoothing=wl.smoothing, kda=kda)
    if n_pre:
        for t in gh.flat_steps(wk.TokenStream(wl, seqs).next(n_pre)):
            bo.step(t["q"], t["k"], t["v"], t["g"], t["beta"])
    sts = [lqk.State(dims) for _ in range(2)]
    for st in sts:
        gh.upload_state(st, dims, bo.base, bo.buf_k, bo.buf_u, bo.buf_G, bo.n)
    raw = wk.TokenStream(wl, seqs).next(n_pre + 1)
    dev = runner.upload_tokens({k: v[n_pre:] for k, v in raw.items()}, bf16)
    return dims, N, sts, dev


@pytest.mark.parametrize("d,bits,kda,bf16,n_pre", [
    (d, b, k, f, n) for d, b, k, f in itertools.product(DIMS, BITS, (False, True), (False, True)) for n in (0, 26)])
def test_decode_step_at_matches_decode_step(d, bits, kda, bf16, n_pre):
    """leapquant_decode_step_at (the position given by the caller) against
    leapquant_decode_step on the same state and token: every state buffer and
    the output bit for bit (the same arithmetic; only the load order differs)."""
    dims, N, (st1, st2), dev = _uploaded_pair(d, bits, kda, bf16, n_pre)
    o1 = torch.empty((N, d), dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(o1)
    x = {k: v[0] for k, v in dev.items()}
    lqk.decode_step(dims, st1, x["q"], x["k"], x["v"], x["g"], x["beta"], o1)
    lqk.decode_step_at(dims, st2, n_pre, x["q"], x["k"], x["v"], x["g"], x["beta"], o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for f in lqk.STATE_FIELDS:
        assert torch.equal(getattr(st1, f), getattr(st2, f)), f
    assert int(st2.err.item()) == 0


@pytest.mark.parametrize("kda", (False, True))
def test_decode_step_at_skips_heads_at_another_position(kda):
    """A head whose stored buffer length is not the given position is left as
    it was, its output row unwritten, and LQ_DEVERR_BAD_LEN is set; the other
    heads step exactly as with leapquant_decode_step."""
    n_pre = 5
    dims, N, (st1, st2), dev = _uploaded_pair(128, 8, kda, False, n_pre)
    st2.buf_len[1] = n_pre - 2  # one head of the first sequence at another (valid) position
    before = {f: getattr(st2, f).clone() for f in lqk.STATE_FIELDS}
    o1 = torch.empty((N, 128), dtype=torch.float32, device="cuda")
    o2 = torch.full_like(o1, 7.0)
    x = {k: v[0] for k, v in dev.items()}
    lqk.decode_step(dims, st1, x["q"], x["k"], x["v"], x["g"], x["beta"], o1)  # every head at n_pre
    lqk.decode_step_at(dims, st2, n_pre, x["q"], x["k"], x["v"], x["g"], x["beta"], o2)
    torch.cuda.synchronize()
    assert int(st2.err.item()) == lq_deverr_bad_len()
    assert torch.all(o2[1] == 7.0)
    others = [h for h in range(N) if h != 1]
    assert torch.equal(o2[others], o1[others])
    for f in ("codes", "row_scale", "col_scale", "ent_k", "ent_u", "ent_g", "buf_len"):
        a, b, ref = getattr(st2, f), before[f], getattr(st1, f)
        assert torch.equal(a[1], b[1]), f
        assert torch.equal(a[others], ref[others]), f


def lq_deverr_bad_len():
    import re
    import os
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "leapquant.h")).read()
    return int(re.search(r"#define LQ_DEVERR_BAD_LEN (\d+)", hdr).group(1))


def _close_checks(R, post, bits, smoothing, F, heads):
    rebuilt = np.einsum("nli,nlj->nij", post["comp_k"][heads].astype(np.float64), post["comp_u"][heads]) + R
    err = np.linalg.norm(rebuilt - F, axis=(1, 2)) / np.linalg.norm(F, axis=(1, 2))
    g1 = gh.g1_check(R, post, bits, smoothing, heads)
    return float(err.max()), g1


@pytest.mark.parametrize("d,bits,kda,bf16", list(itertools.product(DIMS, BITS, (False, True), (False, True))))
def test_close_and_encode_every_instantiation(d, bits, kda, bf16):
    # (bf16 activations: the buffered tokens' key rows hold bf16 keys, read by
    # every fold pass)
    wl = _wl(d, kda, bf16, batch=4, heads=2)
    dims = runner.dims_for(wl, bits)
    BH = wl.batch * wl.heads
    heads = np.arange(BH)
    # encode (dense input)
    S0 = wk.initial_states(wl, range(wl.batch))
    dec = runner.Decoder(dims, np.full(wl.batch, dims.w_max), np.zeros(wl.batch, np.int32))
    dbg = torch.zeros((BH, d, d), dtype=torch.float32, device="cuda")
    dec.encode(runner.states_to_device(S0), dbg)
    post = gh.download_state(dec.state, dims)
    err, g1 = _close_checks(gh.T(dbg.cpu().numpy()), post, bits, wl.smoothing, S0.reshape(-1, d, d), heads)
    print("encode", d, bits, kda, bf16, err, g1)
    assert err <= 1e-6
    assert g1["same"] >= 0.9999 and g1["max_diff"] <= 1 and g1["s_exact"] and g1["c_ulps"] <= 2.0
    # 21 tokens, then the close: entries r + 21 = 25 (d = 128 stages 20 rows, then 5; d < 128
    # stages 32 at once)
    n_tok = 21
    dev = runner.upload_tokens(wk.TokenStream(wl).next(n_tok), bf16)
    for i in range(n_tok):
        dec.step(dev["q"][i], dev["k"][i], dev["v"][i], dev["g"][i], dev["beta"][i], close=False)
    pre = gh.download_state(dec.state, dims)
    assert np.all(pre["buf_len"] == n_tok)
    F = lq.fold_window(lq.decode(gh.encoded_of(pre)), pre["buf_k"], pre["buf_u"], pre["buf_g"], pre["buf_len"], kda)
    dbg.zero_()
    lqk.window_close(dims, dec.state, None, 0, dbg)
    post = gh.download_state(dec.state, dims)
    err, g1 = _close_checks(gh.T(dbg.cpu().numpy()), post, bits, wl.smoothing, F, heads)
    print("close", d, bits, kda, bf16, err, g1)
    assert err <= 1e-6
    assert g1["same"] >= 0.9999 and g1["max_diff"] <= 1 and g1["s_exact"] and g1["c_ulps"] <= 2.0
    assert np.all(post["buf_len"] == 0) and np.all(post["comp_g"] == 0)
    assert int(dec.state.err.item()) == 0


@pytest.mark.parametrize("d,kda,bf16", list(itertools.product(DIMS, (False, True), (False, True))))
def test_fp32_baseline_every_instantiation(d, kda, bf16):
    wl = _wl(d, kda, bf16, batch=3, heads=2)
    dims = runner.dims_for(wl)
    S0 = wk.initial_states(wl, range(wl.batch))
    S = runner.states_to_device(S0)
    steps = 8
    raw = wk.TokenStream(wl).next(steps)
    dev = runner.upload_tokens(raw, bf16)
    toks = gh.flat_steps(raw)
    Sref = S0.reshape(-1, d, d).astype(np.float64)
    o = torch.empty((wl.batch * wl.heads, d), dtype=torch.float32, device="cuda")
    worst = 0.0
    for t in range(steps):
        lqk.fp32_baseline_step(dims, S, dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], o)
        Sref, oref, _ = lq.exact_step(Sref, toks[t]["q"], toks[t]["k"], toks[t]["v"], toks[t]["g"],
                                      toks[t]["beta"])
        worst = max(worst, gh.rel_l2(o.cpu().numpy(), oref))
    print(d, kda, bf16, worst)
    assert worst <= 1e-5
    assert gh.rel_l2(gh.T(S.cpu().numpy()), Sref) <= 1e-5

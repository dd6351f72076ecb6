"""GPU parity of the window's last token taken inside its close
(leapquant_decode_close_at through the C ABI): against the oracle (the fold of
the GPU's pre-step buffers, then the exact gated-delta step, then G1 + G2 on
the close) and against the two-launch path (leapquant_decode_step_at, then
leapquant_window_close) on the same state and inputs."""
import numpy as np
import pytest
import torch

from linear_attention_recurrent_kda_amd import leapquant as lqk
from linear_attention_recurrent_kda_amd import runner
from linear_attention_recurrent_kda_amd import workloads as wk
from oracle import leapquant_oracle as lq
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

W = wk.WORKLOADS

CASES = [
    ("qwen_gdn", 8, {}),                                   # bf16 activations
    ("qwen_gdn", 8, dict(window=32)),                      # bf16 buffered keys over two fold passes
    ("qwen_gdn", 8, dict(act_bf16=False)),
    ("qwen_gdn", 6, {}),
    ("kda_int4", 4, {}),                                   # per-channel decay, fp32 activations
    ("kda_int4", 8, dict(act_bf16=True)),
    ("kda_int4", 6, {}),
    ("tiny_gdn", 8, {}),                                   # d = 32
    ("tiny_gdn", 4, dict(d_k=64, d_v=64, kda=True)),      # d = 64
    ("tiny_gdn", 6, dict(d_k=64, d_v=64, window=5)),      # a short window
]


def _setup(name, bits, kw):
    base = W[name].replace(**kw) if kw else W[name]
    wl = base.replace(batch=min(base.batch, 4))
    dims = runner.dims_for(wl, bits)
    n = wl.w_max - 1  # the window's last token
    dec = runner.Decoder(dims, np.full(wl.batch, wl.w_max), np.zeros(wl.batch, np.int32))
    dec.encode(runner.states_to_device(wk.initial_states(wl, range(wl.batch))))
    raw = wk.TokenStream(wl).next(n + 1)
    dev = runner.upload_tokens(raw, wl.act_bf16)
    for i in range(n):
        dec.step(dev["q"][i], dev["k"][i], dev["v"][i], dev["g"][i], dev["beta"][i], close=False)
    tok = {k_: v_[n] for k_, v_ in dev.items()}
    last = gh.flat_steps({k_: v_[n:] for k_, v_ in raw.items()})[0]
    return wl, dims, n, dec.state, tok, last


def _clone(dims, st):
    c = lqk.State(dims)
    for f in lqk.STATE_FIELDS:
        getattr(c, f).copy_(getattr(st, f))
    return c


@pytest.mark.parametrize("name,bits,kw", CASES)
def test_decode_close_matches_oracle_and_two_launches(name, bits, kw):
    wl, dims, n, st, tok, last = _setup(name, bits, kw)
    N, d = wl.batch * wl.heads, wl.d_k
    st2 = _clone(dims, st)
    pre = gh.download_state(st, dims)
    assert np.all(pre["buf_len"] == n)
    o = torch.empty((N, d), dtype=torch.float32, device="cuda")
    dbg = torch.zeros((N, d, d), dtype=torch.float32, device="cuda")
    lqk.decode_close_at(dims, st, n, tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"], o, dbg)
    post = gh.download_state(st, dims)
    assert int(st.err.item()) == 0
    # oracle: the fold of the pre-step buffers, then the token's exact step
    F = lq.fold_window(lq.decode(gh.encoded_of(pre)), pre["buf_k"], pre["buf_u"], pre["buf_g"], pre["buf_len"],
                       wl.kda)
    S_t, o_ref, _ = lq.exact_step(F, last["q"], last["k"], last["v"], last["g"], last["beta"])
    o_gpu = o.cpu().numpy()
    worst_o = max(gh.rel_l2(o_gpu[h], o_ref[h]) for h in range(N))
    # G2: compensators plus the residual rebuild the state after the token
    R = gh.T(dbg.cpu().numpy())
    rebuilt = np.einsum("nli,nlj->nij", post["comp_k"].astype(np.float64), post["comp_u"]) + R
    err = np.linalg.norm(rebuilt - S_t, axis=(1, 2)) / np.linalg.norm(S_t, axis=(1, 2))
    # G1: codes against the oracle's quantisation of the GPU's residual
    g1 = gh.g1_check(R, post, bits, wl.smoothing)
    # the two-launch path on the same state and inputs
    o2 = torch.empty_like(o)
    lqk.decode_step_at(dims, st2, n, tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"], o2)
    lqk.window_close(dims, st2)
    post2 = gh.download_state(st2, dims)
    o2_gpu = o2.cpu().numpy()
    worst_o2 = max(gh.rel_l2(o_gpu[h], o2_gpu[h]) for h in range(N))
    same2 = float(np.mean(post["C"] == post2["C"]))
    diff2 = int(np.max(np.abs(post["C"].astype(np.int64) - post2["C"])))
    print(name, bits, kw, "o vs oracle", worst_o, "vs two launches", worst_o2, "rebuild", err.max(), g1,
          "codes same as two launches", same2, "max diff", diff2)
    assert worst_o <= 1e-5 and worst_o2 <= 1e-5
    assert err.max() <= 1e-6
    assert g1["same"] >= 0.9999 and g1["max_diff"] <= 1 and g1["s_exact"] and g1["c_ulps"] <= 2.0
    assert same2 >= 0.999 and diff2 <= 1
    assert np.all(post["buf_len"] == 0) and np.all(post["comp_g"] == 0)


def test_decode_close_skips_heads_at_another_position():
    """A head whose stored buffer length is not the given position keeps its
    state and output untouched, and LQ_DEVERR_BAD_LEN is raised."""
    wl, dims, n, st, tok, _ = _setup("kda_int4", 4, {})
    N, d = wl.batch * wl.heads, wl.d_k
    st.buf_len[3] = n - 1
    pre = gh.download_state(st, dims)
    o = torch.full((N, d), 7.0, dtype=torch.float32, device="cuda")
    lqk.decode_close_at(dims, st, n, tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"], o)
    post = gh.download_state(st, dims)
    assert int(st.err.item()) & lqk.LQ_DEVERR_BAD_LEN
    for f in ("codes", "row_scale", "col_scale", "ent_k", "ent_u", "ent_g", "buf_len"):
        assert np.array_equal(post[f][3], pre[f][3]), f
    assert torch.all(o[3] == 7.0)
    others = np.arange(N) != 3
    assert np.all(post["buf_len"][others] == 0)
    assert torch.all(torch.isfinite(o[torch.as_tensor(others, device="cuda")]))

"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Protocol (tolerances are the ones the method's target states):
  G1 codes, staged: the oracle smooths and quantises (fp64) the GPU's own
     pre-quantisation residual; codes >= 99.99% identical and all within one
     LSB, key-row scales bit-identical, value-column scales within 2 ulp.
  G2 decomposition: the GPU's compensators plus residual rebuild the dense
     state (the initial state, or the oracle's fold of the GPU's pre-close
     buffers) to <= 1e-6 relative Frobenius.
  G3 outputs: teacher-forced (every window starts from the oracle's
     encoding), every token <= 1e-3 relative L2 over all checked heads and for
     each head; free-running, every token and head within the bound that the
     GPU's and the oracle's window-start states allow (see the test), with
     every close checked against the oracle's close of the same buffers.
  G4 single step from an oracle-made state uploaded bit-exactly: o_t and u_t
     <= 1e-5 relative.
Full-size workloads run the whole batch on the GPU; the oracle checks all
heads of the listed sequences.
"""
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


def _subset(wl):
    B = wl.batch
    return sorted({0, 1, 2, 3, B - 2, B - 1} & set(range(B)))


def _encode_case(wl, bits):
    dims = runner.dims_for(wl, bits)
    st = lqk.State(dims)
    S0 = wk.initial_states(wl, range(wl.batch))
    dbg = torch.empty((wl.batch * wl.heads, wl.d_v, wl.d_k), dtype=torch.float32, device="cuda")
    lqk.encode(dims, runner.states_to_device(S0), st, dbg)
    host = gh.download_state(st, dims)
    R = gh.T(dbg.cpu().numpy())
    return dims, S0.reshape(-1, wl.d_k, wl.d_v), host, R


@pytest.mark.parametrize("name,bits", [("tiny_gdn", 8), ("qwen_gdn", 8), ("kda_int4", 4), ("kda_int4", 8),
                                       ("qwen_gdn", 6), ("tiny_gdn", 6)])
def test_encode_codes_and_decomposition(name, bits):
    wl = W[name]
    if name == "kda_int4":
        wl = wl.replace(batch=16)
    dims, S0, host, R = _encode_case(wl, bits)
    g1 = gh.g1_check(R, host, bits, wl.smoothing)
    print(name, bits, g1)
    assert g1["same"] >= 0.9999 and g1["max_diff"] <= 1
    assert g1["s_exact"] and g1["c_ulps"] <= 2.0
    # G2: compensators + residual rebuild the initial state
    rebuilt = np.einsum("nli,nlj->nij", host["comp_k"].astype(np.float64), host["comp_u"]) + R
    err = np.linalg.norm(rebuilt - S0, axis=(1, 2)) / np.linalg.norm(S0, axis=(1, 2))
    assert err.max() <= 1e-6, err.max()
    assert np.all(host["buf_len"] == 0)
    # the compensators follow the oracle's power method (same start vectors)
    ref = lq.encode(S0.astype(np.float64), wl.n_comp, wl.power_iters, bits, wl.smoothing)
    cos = np.abs(np.einsum("nli,nli->nl", host["comp_k"].astype(np.float64), ref.comp_k))
    assert cos.min() >= 1 - 1e-4, cos.min()
    # end-to-end code agreement is reported, not gated
    print("end-to-end code agreement", float(np.mean(host["C"] == ref.codes)))


@pytest.mark.parametrize("name,bits", [("tiny_gdn", 8), ("kda_int4", 4), ("qwen_gdn", 6), ("tiny_gdn", 6)])
def test_dequantize_matches_oracle_decode(name, bits):
    wl = W[name].replace(batch=min(W[name].batch, 4))
    dims, S0, host, R = _encode_case(wl, bits)
    out = torch.empty((wl.batch * wl.heads, wl.d_v, wl.d_k), dtype=torch.float32, device="cuda")
    lqk.dequantize(dims, lqk_state_from_host(dims, host), out)
    ref = lq.decode(gh.encoded_of(host))
    assert gh.rel_l2(gh.T(out.cpu().numpy()), ref) <= 1e-6


def lqk_state_from_host(dims, host):
    st = lqk.State(dims)
    for n in lqk.STATE_FIELDS:
        getattr(st, n).copy_(torch.from_numpy(host[n]))
    return st


@pytest.mark.parametrize("name,bits,n_pre", [("tiny_gdn", 8, 5), ("qwen_gdn", 8, 7), ("kda_int4", 4, 9),
                                              ("kda_int4", 8, 0), ("prefix_mix", 8, 20), ("qwen_gdn", 6, 7),
                                              ("kda_int4", 6, 9)])
def test_single_step_from_uploaded_state(name, bits, n_pre):
    """G4: oracle state after n_pre buffered tokens, rounded to fp32 and uploaded."""
    wl = W[name]
    seqs = list(range(min(wl.batch, 4)))
    wl = wl.replace(batch=len(seqs))
    H, d = wl.heads, wl.d_k
    dims = runner.dims_for(wl, bits)
    S0 = wk.initial_states(wl, seqs).reshape(-1, d, d).astype(np.float64)
    stream = wk.TokenStream(wl, seqs)
    toks = gh.flat_steps(stream.next(n_pre + 1))
    N = len(seqs) * H
    bo = lq.BufferedOracle(S0, np.full(N, 10 ** 6), np.zeros(N), w_max=wl.w_max, r=wl.n_comp,
                           T=wl.power_iters, bits=bits, smoothing=wl.smoothing, kda=wl.kda)
    for t in toks[:n_pre]:
        bo.step(t["q"], t["k"], t["v"], t["g"], t["beta"])
    # round the whole state to fp32, as it will sit on the GPU
    r32 = lambda x: np.asarray(x, np.float32).astype(np.float64)
    for f in ("comp_k", "comp_u", "s", "c"):
        setattr(bo.base, f, r32(getattr(bo.base, f)))
    bo.buf_k, bo.buf_u, bo.buf_G = r32(bo.buf_k), r32(bo.buf_u), r32(bo.buf_G)
    st = lqk.State(dims)
    gh.upload_state(st, dims, bo.base, bo.buf_k, bo.buf_u, bo.buf_G, bo.n)
    last = toks[n_pre]
    o_ref, u_ref = bo.step(last["q"], last["k"], last["v"], last["g"], last["beta"])
    raw = wk.TokenStream(wl, seqs).next(n_pre + 1)
    dev = runner.upload_tokens({k: v[n_pre:] for k, v in raw.items()}, wl.act_bf16)
    o = torch.empty((N, d), dtype=torch.float32, device="cuda")
    lqk.decode_step(dims, st, dev["q"][0], dev["k"][0], dev["v"][0], dev["g"][0], dev["beta"][0], o)
    host = gh.download_state(st, dims)
    u_gpu = host["buf_u"][np.arange(N), n_pre]
    print(name, bits, gh.rel_l2(o.cpu().numpy(), o_ref), gh.rel_l2(u_gpu, u_ref))
    assert gh.rel_l2(o.cpu().numpy(), o_ref) <= 1e-5
    assert gh.rel_l2(u_gpu, u_ref) <= 1e-5
    assert np.all(host["buf_len"] == n_pre + 1)
    assert np.array_equal(host["buf_k"][np.arange(N), n_pre], np.asarray(last["k"], np.float32))


G3_CASES = [
    ("tiny_gdn", 8, 64, {}),
    ("tiny_gdn", 8, 24, dict(batch=2, heads=2, window=1, n_comp=0)),   # per-token requantisation
    ("qwen_gdn", 8, 256, {}),
    ("serving_gdn", 8, 48, {}),
    ("kda_int4", 4, 48, {}),
    ("kda_int4", 8, 48, {}),
    ("prefix_mix", 8, 64, {}),
    ("qwen_gdn", 6, 64, {}),
    ("kda_int4", 6, 48, {}),
    ("kda_int4", 4, 48, dict(act_bf16=True)),   # per-channel decay with bf16 activations
    ("prefix_mix", 8, 64, dict(act_bf16=True)),  # staggered windows, bf16 buffered keys, close lists
]


def _g3_setup(name, kw):
    wl = W[name].replace(**kw) if kw else W[name]
    seqs = list(range(wl.batch)) if wl.batch * wl.heads <= 256 else _subset(wl)
    return wl, seqs


def _per_head(o, ref, d_v):
    """Relative L2 of each head's output at each step: [steps][heads]."""
    a = np.asarray(o, np.float64).reshape(o.shape[0], -1, d_v)
    b = np.asarray(ref, np.float64).reshape(a.shape)
    return np.linalg.norm(a - b, axis=2) / np.linalg.norm(b, axis=2)


@pytest.mark.parametrize("name,bits,steps,kw", G3_CASES)
def test_outputs_teacher_forced(name, bits, steps, kw):
    """G3, teacher-forced: at every window start the checked heads hold the
    oracle's encoding; every token's output must then match to 1e-3, over all
    checked heads together and for every head on its own."""
    wl, seqs = _g3_setup(name, kw)
    ref = gh.run_oracle(wl, steps, seqs, bits, record=True)
    o_gpu, _, err = gh.run_gpu(wl, steps, seqs, bits, force=ref)
    assert err == 0
    per_step = [gh.rel_l2(o_gpu[t], ref["o"][t]) for t in range(steps)]
    head = _per_head(o_gpu, ref["o"], wl.d_v)
    t_w, h_w = np.unravel_index(np.argmax(head), head.shape)
    print(name, bits, kw, "teacher-forced max rel L2", max(per_step), "at", int(np.argmax(per_step)),
          "| worst head", head.max(), "(step", int(t_w), "head", int(h_w), ")")
    assert max(per_step) <= 1e-3
    assert head.max() <= 1e-3


# Relative noise on a close's input (16 fp32 ulps) at which the oracle's own
# codes are reported beside the GPU's: how many codes the GPU's close sets
# differently from the oracle's close of the same buffers, against how many
# the oracle itself sets differently under this noise. Reported, not gated:
# with a fixed small number of power iterations the fp32 and fp64
# compensators of a nearly degenerate head can differ enough to move a row of
# codes, in the GPU and in the noisy oracle alike.
FLIP_NOISE = 2.0 ** -20


@pytest.mark.parametrize("name,bits,steps,kw", G3_CASES)
def test_outputs_free_running(name, bits, steps, kw):
    """G3, free-running from the same initial state, split into the two things
    the run is made of.

    (a) Windows. Inside a window both sides run the exact recurrence from their
    own window-start state (the GPU in the buffered form, in fp32). The
    recurrence is affine in the state, S_t = A_t S_c + B_t, with the same B_t on
    both sides and A_t a product of (I - beta k k^T) Diag(alpha) factors: decay
    alpha <= 1 and 0 < beta |k|^2 < 2 give |A_t|_2 <= 1. A window-start
    difference therefore never grows inside the window, and for every head and
    token |o_gpu - o_ref| <= |Dec_gpu - Dec_ref|_2 |q_t| + 1e-3 |o_ref|, the
    window start being the head's last close (or the initial encode) on each
    side and 1e-3 the output tolerance for the window's own arithmetic.
    (b) Closes. Every close the GPU makes passes G1 and G2 on its own
    pre-close buffers: its compensators plus the residual it quantized rebuild
    the oracle's fold of those buffers within 1e-6, and its codes and scales
    are the oracle's quantization of that residual (codes >= 99.99% identical,
    all within one LSB; row scales bit-identical; column scales within 2 ulp).
    Rounding decisions at near-ties are where the two runs part (a code flip
    persists, [article] on per-step quantization); (a) and (b) together account
    for every difference, with no free factor."""
    wl, seqs = _g3_setup(name, kw)
    r, T = wl.n_comp, wl.power_iters
    ref = gh.run_oracle(wl, steps, seqs, bits, record=True)
    ref_close = {ev.step: ev for ev in ref["closes"]}
    rng = np.random.default_rng(5)
    tally = dict(flips=0, l1=0, noisy_l1=0, codes=0, off_by_more=0, g2=0.0, g1_same=1.0)
    events = []  # (step, local heads, |Dec_gpu - Dec_ref|_2 of those heads)

    def on_close(t, local, pre, post, R):
        F = lq.fold_window(lq.decode(gh.encoded_of(pre)), pre["buf_k"], pre["buf_u"], pre["buf_g"],
                           pre["buf_len"], wl.kda)
        # (b): G2 and G1 of this close
        rebuilt = np.einsum("nli,nlj->nij", post["comp_k"].astype(np.float64), post["comp_u"]) + R
        g2 = float((np.linalg.norm(rebuilt - F, axis=(1, 2)) / np.linalg.norm(F, axis=(1, 2))).max())
        g1 = gh.g1_check(R, post, bits, wl.smoothing)
        assert g2 <= 1e-6, (t, g2)
        assert g1["same"] >= 0.9999 and g1["max_diff"] <= 1 and g1["s_exact"] and g1["c_ulps"] <= 2.0, (t, g1)
        tally["g2"] = max(tally["g2"], g2)
        tally["g1_same"] = min(tally["g1_same"], g1["same"])
        # reported: end-to-end code changes against the oracle's close of the same buffers
        start = pre["comp_u"] if wl.warm_start else None  # the variant starts from the closing window's
        e = lq.encode(F, r, T, bits, wl.smoothing, start=start)
        diff = np.abs(post["C"] - e.codes)
        tally["flips"] += int(np.count_nonzero(diff))
        tally["l1"] += int(diff.sum())
        tally["off_by_more"] += int(np.count_nonzero(diff > 1))
        tally["codes"] += diff.size
        en = lq.encode(F * (1.0 + FLIP_NOISE * rng.standard_normal(F.shape)), r, T, bits, wl.smoothing,
                       start=start)
        tally["noisy_l1"] += int(np.abs(en.codes - e.codes).sum())
        # (a): the window-start difference against the free-running oracle's window start
        ev = ref_close[t]
        assert np.array_equal(np.sort(ev.heads), np.sort(local))
        D_ref = lq.decode(ev.enc.take(np.argsort(ev.heads)))
        D_gpu = lq.decode(gh.encoded_of(post).take(np.argsort(local)))
        events.append((t, np.sort(local), np.linalg.norm(D_gpu - D_ref, ord=2, axis=(1, 2))))

    o_gpu, _, err, start = gh.run_gpu_closes(wl, steps, seqs, bits, on_close)
    assert err == 0
    N, d_v = len(seqs) * wl.heads, wl.d_v
    # window-start difference in force at each step (a close after step t acts from t + 1)
    delta = np.linalg.norm(lq.decode(gh.encoded_of(start)) - lq.decode(ref["enc0"]), ord=2, axis=(1, 2))
    delta_t = np.empty((steps, N))
    ev_at = {t: (loc, dl) for (t, loc, dl) in events}
    for t in range(steps):
        delta_t[t] = delta
        if t in ev_at:
            loc, dl = ev_at[t]
            delta = delta.copy()
            delta[loc] = dl
    toks = gh.flat_steps(wk.TokenStream(wl, seqs).next(steps))
    qn = np.stack([np.linalg.norm(tk["q"], axis=1) for tk in toks])             # [steps][N]
    og = o_gpu.reshape(steps, N, d_v).astype(np.float64)
    orf = ref["o"].reshape(steps, N, d_v)
    dist = np.linalg.norm(og - orf, axis=2)
    bound = delta_t * qn + 1e-3 * np.linalg.norm(orf, axis=2)
    head = dist / np.linalg.norm(orf, axis=2)
    err_t = np.array([gh.rel_l2(o_gpu[t], ref["o"][t]) for t in range(steps)])
    print(name, bits, kw, "free-running max rel L2", err_t.max(), "at", int(err_t.argmax()),
          "| worst head", head.max(), "| max distance / bound", (dist / bound).max(),
          "| closes", len(events), "max G2", tally["g2"], "min G1 same", tally["g1_same"],
          "| end to end: codes changed", tally["flips"], "of", tally["codes"],
          "(by more than one LSB:", tally["off_by_more"], ") sum |dC|", tally["l1"], "; oracle at noise",
          FLIP_NOISE, ": sum |dC|", tally["noisy_l1"])
    assert np.all(dist <= bound)


@pytest.mark.parametrize("name,bits,n_tok,close_seqs,kw", [
    ("qwen_gdn", 8, 16, None, {}),          # full window, every sequence
    ("kda_int4", 4, 16, None, {}),
    ("kda_int4", 8, 16, None, {}),
    ("tiny_gdn", 8, 5, [1], {}),            # partial window, one sequence of two
    ("prefix_mix", 8, 11, [0, 3, 5], {}),   # partial windows, a close list
    ("prefix_mix", 8, 11, [0, 3, 5], dict(act_bf16=True)),  # the same with bf16 buffered keys
    ("qwen_gdn", 6, 16, None, {}),
    ("tiny_gdn", 6, 5, [1], {}),            # d = 32: four threads share a low-bit word
    ("tiny_gdn", 6, 7, [0], dict(d_k=64, d_v=64)),             # d = 64: two threads share it
    ("tiny_gdn", 4, 9, None, dict(d_k=64, d_v=64, kda=True)),
])
def test_close_codes_and_decomposition(name, bits, n_tok, close_seqs, kw):
    """G1 + G2 at a window close: the oracle folds the GPU's pre-close buffers;
    the GPU's compensators plus its residual must rebuild that fold, and its
    codes must match the oracle's quantisation of its own residual."""
    base = W[name].replace(**kw) if kw else W[name]
    wl = base.replace(batch=8 if base.batch >= 8 else base.batch + 1)
    dims = runner.dims_for(wl, bits)
    dec = runner.Decoder(dims, np.full(wl.batch, wl.w_max), np.zeros(wl.batch, np.int32))
    dec.encode(runner.states_to_device(wk.initial_states(wl, range(wl.batch))))
    dev = runner.upload_tokens(wk.TokenStream(wl).next(n_tok), wl.act_bf16)
    for i in range(n_tok):
        dec.step(dev["q"][i], dev["k"][i], dev["v"][i], dev["g"][i], dev["beta"][i], close=False)
    pre = gh.download_state(dec.state, dims)
    assert np.all(pre["buf_len"] == n_tok)
    seqs = list(range(wl.batch)) if close_seqs is None else close_seqs
    heads = gh.heads_of(seqs, wl.heads)
    F = lq.fold_window(lq.decode(gh.encoded_of(pre).take(heads)), pre["buf_k"][heads], pre["buf_u"][heads],
                       pre["buf_g"][heads], pre["buf_len"][heads], wl.kda)
    dbg = torch.zeros((wl.batch * wl.heads, wl.d_v, wl.d_k), dtype=torch.float32, device="cuda")
    ids = None if close_seqs is None else torch.tensor(close_seqs, dtype=torch.int32, device="cuda")
    lqk.window_close(dims, dec.state, ids, 0, dbg)
    post = gh.download_state(dec.state, dims)
    R = gh.T(dbg.cpu().numpy())[heads]
    rebuilt = np.einsum("nli,nlj->nij", post["comp_k"][heads].astype(np.float64), post["comp_u"][heads]) + R
    err = np.linalg.norm(rebuilt - F, axis=(1, 2)) / np.linalg.norm(F, axis=(1, 2))
    assert err.max() <= 1e-6, (name, err.max())
    g1 = gh.g1_check(R, post, bits, wl.smoothing, heads)
    print(name, bits, n_tok, g1)
    assert g1["same"] >= 0.9999 and g1["max_diff"] <= 1 and g1["s_exact"] and g1["c_ulps"] <= 2.0
    closed = np.zeros(wl.batch * wl.heads, bool)
    closed[heads] = True
    assert np.all(post["buf_len"][closed] == 0) and np.all(post["buf_len"][~closed] == n_tok)
    # heads that were not closed are untouched
    for f in ("codes", "row_scale", "col_scale", "ent_k", "ent_u", "ent_g"):
        assert np.array_equal(post[f][~closed], pre[f][~closed]), f
    # compensators sit at window position 0 (G = 0)
    assert np.all(post["comp_g"][heads] == 0)


@pytest.mark.parametrize("name", ["tiny_gdn", "qwen_gdn", "kda_int4"])
def test_fp32_baseline_matches_exact_recurrence(name):
    wl = W[name].replace(batch=min(W[name].batch, 8))
    dims = runner.dims_for(wl)
    S0 = wk.initial_states(wl, range(wl.batch))
    S = runner.states_to_device(S0)
    steps = 24
    raw = wk.TokenStream(wl).next(steps)
    dev = runner.upload_tokens(raw, wl.act_bf16)
    toks = gh.flat_steps(raw)
    Sref = S0.reshape(-1, wl.d_k, wl.d_v).astype(np.float64)
    o = torch.empty((wl.batch * wl.heads, wl.d_v), dtype=torch.float32, device="cuda")
    for t in range(steps):
        lqk.fp32_baseline_step(dims, S, dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], o)
        Sref, oref, _ = lq.exact_step(Sref, toks[t]["q"], toks[t]["k"], toks[t]["v"], toks[t]["g"],
                                      toks[t]["beta"])
        assert gh.rel_l2(o.cpu().numpy(), oref) <= 1e-5
    assert gh.rel_l2(gh.T(S.cpu().numpy()), Sref) <= 1e-5


def test_deterministic():
    wl = W["qwen_gdn"].replace(batch=8)
    a, dec_a, _ = gh.run_gpu(wl, 40, list(range(8)))
    b, dec_b, _ = gh.run_gpu(wl, 40, list(range(8)))
    assert np.array_equal(a, b)
    for n in lqk.STATE_FIELDS:
        assert torch.equal(getattr(dec_a.state, n), getattr(dec_b.state, n)), n


def test_power_of_two_scaling_is_exact():
    wl = W["qwen_gdn"].replace(batch=4)
    dims = runner.dims_for(wl)
    S0 = wk.initial_states(wl, range(4))
    outs = []
    for p in (0, 5):
        st = lqk.State(dims)
        lqk.encode(dims, runner.states_to_device(S0 * np.float32(2.0 ** p)), st)
        outs.append(gh.download_state(st, dims))
    a, b = outs
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["row_scale"] * np.float32(32.0), b["row_scale"])
    assert np.array_equal(a["col_scale"], b["col_scale"])
    assert np.array_equal(a["comp_k"], b["comp_k"])
    assert np.array_equal(a["comp_u"] * np.float32(32.0), b["comp_u"])


@pytest.mark.parametrize("kda", [False, True])
def test_max_window_and_compensators(kda):
    """w_max = 64 with r = 8: more entries than the decode step prefetches (24)
    and than one fold pass of the close (16), for both decays."""
    wl = W["tiny_gdn"].replace(batch=2, heads=3, d_k=128, d_v=128, window=64, n_comp=8, steps=70, kda=kda)
    steps = 70
    ref = gh.run_oracle(wl, steps, [0, 1], record=True)
    o_gpu, _, err = gh.run_gpu(wl, steps, [0, 1], force=ref)  # teacher-forced: the arithmetic alone
    assert err == 0
    head = _per_head(o_gpu, ref["o"], wl.d_v)
    print("kda", kda, "worst head rel L2", head.max())
    assert head.max() <= 1e-3


@pytest.mark.parametrize("d,kda,bits", [(64, False, 8), (64, True, 8), (32, True, 8), (64, False, 6), (64, True, 4),
                                         (32, False, 4), (32, True, 6)])
def test_other_head_dims(d, kda, bits):
    """Outputs over 40 tokens (two closes) at d = 32 and 64, teacher-forced (G3):
    the code layouts and the close's cross-thread low-bit words of the narrower
    heads."""
    wl = W["tiny_gdn"].replace(batch=3, heads=2, d_k=d, d_v=d, kda=kda, steps=40)
    ref = gh.run_oracle(wl, 40, [0, 1, 2], bits, record=True)
    o_gpu, _, err = gh.run_gpu(wl, 40, [0, 1, 2], bits, force=ref)
    assert err == 0
    assert max(gh.rel_l2(o_gpu[t], ref["o"][t]) for t in range(40)) <= 1e-3


@pytest.mark.parametrize("kda", [False, True])
def test_close_skips_heads_with_a_corrupted_length(kda):
    """A head whose stored buffer length lies outside [0, w_max] is left
    untouched by the close (its fold runs on the length clamped into range,
    and the check comes before any write) and LQ_DEVERR_BAD_LEN is raised;
    the other heads close."""
    wl = W["tiny_gdn"].replace(batch=2, heads=2, window=6, kda=kda)
    dims = runner.dims_for(wl)
    dec = runner.Decoder(dims, np.full(wl.batch, wl.w_max), np.zeros(wl.batch, np.int32))
    dec.encode(runner.states_to_device(wk.initial_states(wl, range(wl.batch))))
    dev = runner.upload_tokens(wk.TokenStream(wl).next(4), False)
    for i in range(4):
        dec.step(dev["q"][i], dev["k"][i], dev["v"][i], dev["g"][i], dev["beta"][i], close=False)
    st = dec.state
    st.buf_len[1] = dims.w_max + 3
    st.buf_len[2] = -1
    pre = gh.download_state(st, dims)
    lqk.window_close(dims, st)
    post = gh.download_state(st, dims)
    assert int(st.err.item()) & lqk.LQ_DEVERR_BAD_LEN
    for h in (1, 2):
        for f in ("codes", "row_scale", "col_scale", "ent_k", "ent_u", "ent_g", "buf_len"):
            assert np.array_equal(post[f][h], pre[f][h]), (h, f)
    assert post["buf_len"][0] == 0 and post["buf_len"][3] == 0
    assert not np.array_equal(post["codes"][0], pre["codes"][0])


def test_device_error_flags_and_empty_call():
    wl = W["tiny_gdn"].replace(batch=2, heads=2, window=4)
    dims = runner.dims_for(wl)
    st = lqk.State(dims)
    lqk.encode(dims, runner.states_to_device(wk.initial_states(wl, [0, 1])), st)
    st.buf_len[1] = dims.w_max  # host forces the buffer-full precondition on head 1
    before = {n: getattr(st, n).clone() for n in ("buf_k", "buf_u", "buf_g")}
    dev = runner.upload_tokens(wk.TokenStream(wl).next(1), False)
    o = torch.full((4, 32), 7.0, device="cuda")
    lqk.decode_step(dims, st, dev["q"][0], dev["k"][0], dev["v"][0], dev["g"][0], dev["beta"][0], o)
    torch.cuda.synchronize()
    assert int(st.err.item()) & lqk.LQ_DEVERR_BUFFER_FULL
    assert torch.all(o[1] == 7.0) and not torch.all(o[0] == 7.0)
    assert int(st.buf_len[1]) == dims.w_max and int(st.buf_len[0]) == 1
    for n, t in before.items():
        assert torch.equal(getattr(st, n)[1], t[1])
    st.err.zero_()
    lqk.window_close(dims, st, torch.tensor([5], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int(st.err.item()) & lqk.LQ_DEVERR_BAD_SEQ
    # empty batch: accepted, nothing enqueued
    lqk.decode_step(runner.dims_for(wl.replace(batch=0)), lqk.State(runner.dims_for(wl.replace(batch=0))),
                    dev["q"][0], dev["k"][0], dev["v"][0], dev["g"][0], dev["beta"][0], o)

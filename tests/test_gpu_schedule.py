"""The overlapped layer schedule (runner.capture_tokens with overlap=True: the
window close of layer l on a side stream beside the other layers' decodes)
against the plain eager order, on a stack of layers: every state buffer and the
last outputs must be bit-identical, on every one of several graph replays
(with eager work between them). The schedule only reorders independent work,
so equality is exact."""
import numpy as np
import pytest
import torch

from linear_attention_recurrent_kda_amd import leapquant as lqk
from linear_attention_recurrent_kda_amd import runner
from linear_attention_recurrent_kda_amd import workloads as wk

pytestmark = pytest.mark.gpu

W = wk.WORKLOADS


@pytest.mark.parametrize("name,kw,L,T", [("qwen_gdn", dict(batch=8), 3, 40),
                                          ("prefix_mix", dict(batch=6), 2, 40),
                                          ("kda_int4", dict(batch=4), 2, 20)])
def test_overlapped_schedule_matches_eager(name, kw, L, T):
    wl = W[name].replace(**kw)
    dims = runner.dims_for(wl)
    S0 = runner.states_to_device(wk.initial_states(wl, range(wl.batch)))
    inputs = [wk.device_tokens(wl, T, seed=l) for l in range(L)]
    BH = wl.batch * wl.heads

    def fresh():
        decs = [runner.Decoder(dims, wk.window_lengths(wl), wk.window_offsets(wl)) for _ in range(L)]
        for d in decs:
            d.encode(S0)
        return decs

    # eager reference: layer by layer per token, closes after the token
    ref = fresh()
    ref_out = [torch.empty((BH, wl.d_v), device="cuda") for _ in range(L)]
    for t in range(T):
        for l, d in enumerate(ref):
            x = inputs[l]
            lqk.decode_step(dims, d.state, x["q"][t], x["k"][t], x["v"][t], x["g"][t], x["beta"][t], ref_out[l])
        for d in ref:
            d.close_due(t)
    torch.cuda.synchronize()
    want = [{f: getattr(d.state, f).clone() for f in lqk.STATE_FIELDS} for d in ref]
    assert sum(d.closes_at(t) for t in range(T) for d in ref) > 0

    decs = fresh()
    outs = [torch.empty((BH, wl.d_v), device="cuda") for _ in range(L)]
    g = runner.capture_tokens(decs, inputs, outs, 0, T, overlap=True)
    for rep in range(3):
        for d in decs:  # eager work between replays: back to the encoded start
            d.encode(S0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l, d in enumerate(decs):
            for f in lqk.STATE_FIELDS:
                assert torch.equal(getattr(d.state, f), want[l][f]), (rep, l, f)
            assert torch.equal(outs[l], ref_out[l]), (rep, l)

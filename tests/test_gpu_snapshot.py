"""Prefix-cache snapshots through the C ABI: a window-boundary state survives
snapshot + restore bit for bit and decodes on identically; heads inside a
window are refused."""
import numpy as np
import pytest
import torch

from linear_attention_recurrent_kda_amd import leapquant as lqk
from linear_attention_recurrent_kda_amd import runner
from linear_attention_recurrent_kda_amd import workloads as wk
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

W = wk.WORKLOADS


@pytest.mark.parametrize("name,bits", [("qwen_gdn", 8), ("kda_int4", 4), ("tiny_gdn", 6)])
def test_snapshot_restore_round_trip(name, bits):
    wl = W[name].replace(batch=4)
    dims = runner.dims_for(wl, bits)
    H, N, d = wl.heads, 4 * wl.heads, wl.d_k
    W_ = wl.w_max
    dec = runner.Decoder(dims, np.full(4, W_), np.zeros(4, np.int32))
    dec.encode(runner.states_to_device(wk.initial_states(wl, range(4))))
    dev = runner.upload_tokens(wk.TokenStream(wl).next(W_ + 8), wl.act_bf16)
    for t in range(W_):  # one full window: the close leaves every buffer empty
        dec.step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t])
    seqs = [3, 1]
    ids = torch.tensor(seqs, dtype=torch.int32, device="cuda")
    rec = lqk.snapshot_bytes(dims)
    snap = torch.zeros((len(seqs), H, rec), dtype=torch.uint8, device="cuda")
    lqk.snapshot(dims, dec.state, snap, ids)
    fresh = lqk.State(dims)
    fresh.ent_g.fill_(5.0)      # restore must reset the compensator G and the length
    fresh.buf_len.fill_(3)
    lqk.restore(dims, fresh, snap, ids)
    a, b = gh.download_state(dec.state, dims), gh.download_state(fresh, dims)
    heads = gh.heads_of(seqs, H)
    for f in ("codes", "row_scale", "col_scale", "comp_k", "comp_u"):
        assert np.array_equal(a[f][heads], b[f][heads]), f
    assert np.all(b["comp_g"][heads] == 0) and np.all(b["buf_len"][heads] == 0)
    # the record layout as the header states it: codes, s, c, compensator keys, values
    host = snap.cpu().numpy()
    for slot, seq in enumerate(seqs):
        for h in range(H):
            n = seq * H + h
            want = b"".join(np.ascontiguousarray(x).tobytes() for x in (
                a["codes"][n], a["row_scale"][n], a["col_scale"][n], a["comp_k"][n], a["comp_u"][n]))
            assert host[slot, h].tobytes() == want, (seq, h)
    assert int(dec.state.err.item()) == 0 and int(fresh.err.item()) == 0
    # decoding on: the restored heads give the original heads' outputs exactly
    o1 = torch.empty((N, d), device="cuda")
    o2 = torch.empty((N, d), device="cuda")
    for t in range(W_, W_ + 8):
        lqk.decode_step(dims, dec.state, dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], o1)
        lqk.decode_step(dims, fresh, dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], o2)
        idx = torch.as_tensor(heads, device="cuda", dtype=torch.long)
        assert torch.equal(o1[idx], o2[idx])
    # memory accounting: the record is the window-boundary state, far below fp32
    assert rec == d * d * bits // 8 + 8 * d + 8 * wl.n_comp * d
    assert rec < 4 * d * d


def test_snapshot_refuses_heads_inside_a_window():
    wl = W["tiny_gdn"].replace(batch=2, heads=2)
    dims = runner.dims_for(wl)
    st = lqk.State(dims)
    lqk.encode(dims, runner.states_to_device(wk.initial_states(wl, [0, 1])), st)
    dev = runner.upload_tokens(wk.TokenStream(wl).next(1), False)
    o = torch.empty((4, wl.d_v), device="cuda")
    lqk.decode_step(dims, st, dev["q"][0], dev["k"][0], dev["v"][0], dev["g"][0], dev["beta"][0], o)
    rec = lqk.snapshot_bytes(dims)
    snap = torch.full((2, 2, rec), 0xA5, dtype=torch.uint8, device="cuda")
    lqk.snapshot(dims, st, snap)
    torch.cuda.synchronize()
    assert int(st.err.item()) & lqk.LQ_DEVERR_BAD_LEN
    assert torch.all(snap == 0xA5)

"""Test-side helpers for GPU-vs-oracle parity: code (un)packing, token
flattening, and the two runs (HIP path through the C ABI, fp64 oracle) on the
same seeded inputs. Nothing here computes the method: the oracle does that on
the CPU and the HIP kernels on the GPU."""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np
import torch

from linear_attention_recurrent_kda_amd import leapquant as lqk
from linear_attention_recurrent_kda_amd import runner
from linear_attention_recurrent_kda_amd import workloads as wk
from oracle import leapquant_oracle as lq
from tests.oracle_inputs import flat_steps, rel_l2  # noqa: F401


# ---- code format (include/leapquant.h): [BH][d_v][d_k] int8, or int4 packed
def _lo_bits() -> np.ndarray:
    """6-bit codes: bit offset of the 2-bit low field of channel c (0..15) of a
    16-channel group inside its 32-bit word (include/leapquant.h)."""
    c = np.arange(16)
    p = np.where(c % 2 == 0, c // 2, 8 + c // 2)
    return 8 * (p % 4) + 2 * (p // 4)


def _unpack_nibbles(u: np.ndarray) -> np.ndarray:
    """[..][d/2] bytes -> [..][d] signed 4-bit values (channel 2m low nibble)."""
    u = u.astype(np.int32)
    out = np.empty(u.shape[:-1] + (2 * u.shape[-1],), np.int32)
    out[..., 0::2], out[..., 1::2] = ((u & 0xF) ^ 8) - 8, ((u >> 4) ^ 8) - 8
    return out


def _pack_nibbles(x: np.ndarray) -> np.ndarray:
    return ((x[..., 0::2] & 0xF) | ((x[..., 1::2] & 0xF) << 4)).astype(np.uint8)


def unpack_codes(raw: np.ndarray, bits: int, d: int) -> np.ndarray:
    """Device codes [BH][d_v][d_k*bits/8] (bytes) -> math layout [BH][d_k][d_v] int32."""
    raw = np.asarray(raw)
    u = raw.view(np.uint8).reshape(-1, d, d * bits // 8)
    if bits == 8:
        Ct = raw.view(np.int8).reshape(-1, d, d).astype(np.int32)
    elif bits == 4:
        Ct = _unpack_nibbles(u)
    else:
        head = raw.view(np.uint8).reshape(-1, 3 * d * d // 4)
        n, nj = head.shape[0], d // 16
        hi = _unpack_nibbles(head[:, : d * d // 2].reshape(n, d, d // 2))           # [BH][d_v][d_k]
        W = np.ascontiguousarray(head[:, d * d // 2:]).view("<u4").reshape(n, 16, nj, nj)  # [jl][g][jh]
        words = W.transpose(0, 3, 1, 2).reshape(n, d, nj).astype(np.int64)         # [BH][j][g]
        lo = (words[:, :, :, None] >> _lo_bits()[None, None, None, :]) & 3          # [BH][d_v][g][16]
        Ct = 4 * hi + lo.reshape(hi.shape).astype(np.int32)
    return np.ascontiguousarray(np.swapaxes(Ct, 1, 2))


def pack_codes(C: np.ndarray, bits: int) -> np.ndarray:
    """Math layout [BH][d_k][d_v] ints -> device bytes [BH][d_v][d_k*bits/8] (int8)."""
    Ct = np.swapaxes(np.asarray(C, np.int32), 1, 2)
    if bits == 8:
        return np.ascontiguousarray(Ct.astype(np.int8))
    if bits == 4:
        return np.ascontiguousarray(_pack_nibbles(Ct).view(np.int8))
    n, d, _ = Ct.shape
    nj = d // 16
    hi, lo = Ct >> 2, (Ct & 3).astype(np.uint32)
    words = (lo.reshape(n, d, nj, 16) << _lo_bits().astype(np.uint32)).sum(axis=3, dtype=np.uint32)  # [j][g]
    W = words.reshape(n, nj, 16, nj).transpose(0, 2, 3, 1)                        # [jl][g][jh]
    lo_bytes = np.ascontiguousarray(W.astype("<u4")).view(np.uint8).reshape(n, d * d // 4)
    hi_bytes = _pack_nibbles(hi).reshape(n, d * d // 2)
    return np.ascontiguousarray(np.concatenate([hi_bytes, lo_bytes], axis=1).reshape(n, d, 3 * d // 4).view(np.int8))


def T(x: np.ndarray) -> np.ndarray:
    """[..][a][b] -> [..][b][a]."""
    return np.ascontiguousarray(np.swapaxes(x, -1, -2))


def buf_keys_f32(ent_k: np.ndarray, dims: lqk.Dims) -> np.ndarray:
    """Buffered tokens' keys as fp32 [BH][w_max][d] from the entry key rows. With
    bf16 activations a token's key row holds its bf16 key in the row's first
    d * 2 bytes; compensator rows (entries < r) and fp32 rows are fp32."""
    rows = np.ascontiguousarray(ent_k[:, dims.n_comp:], np.float32)
    if not dims.bf16:
        return rows
    raw = rows.view(np.uint16).reshape(rows.shape[0], rows.shape[1], 2 * dims.d)[:, :, :dims.d]
    return wk.bf16_to_f32(raw).reshape(rows.shape)


def buf_key_rows(buf_k, dims: lqk.Dims) -> np.ndarray:
    """fp32 buffered keys [BH][w_max][d] -> the entry key rows' contents (bf16
    activations: the keys must be bf16 values; they fill each row's first half)."""
    k = np.ascontiguousarray(np.asarray(buf_k, np.float32))
    if not dims.bf16:
        return k
    bits = wk.round_to_bf16(k)
    assert np.array_equal(wk.bf16_to_f32(bits), k), "buffered keys with bf16 activations must be bf16 values"
    raw = np.zeros(k.shape[:-1] + (2 * dims.d,), np.uint16)
    raw[..., :dims.d] = bits
    return raw.view(np.float32).reshape(k.shape)


def download_state(st: lqk.State, dims: lqk.Dims) -> Dict[str, np.ndarray]:
    torch.cuda.synchronize()
    out = {n: getattr(st, n).cpu().numpy() for n in lqk.STATE_FIELDS}
    out["C"] = unpack_codes(out["codes"], dims.bits, dims.d)
    r = dims.n_comp  # entries 0..r-1 are the compensators, the rest the token buffer
    out["comp_k"], out["comp_u"], out["comp_g"] = out["ent_k"][:, :r], out["ent_u"][:, :r], out["ent_g"][:, :r]
    out["buf_k"], out["buf_u"], out["buf_g"] = buf_keys_f32(out["ent_k"], dims), out["ent_u"][:, r:], out["ent_g"][:, r:]
    return out


def encoded_of(host: Dict[str, np.ndarray]) -> lq.Encoded:
    """GPU window-start state as the oracle's Encoded (fp32 values exact in fp64)."""
    f = lambda x: np.asarray(x, np.float64)
    return lq.Encoded(f(host["comp_k"]), f(host["comp_u"]), f(host["row_scale"]), f(host["col_scale"]),
                      host["C"], None, True)


def upload_state(st: lqk.State, dims: lqk.Dims, enc: lq.Encoded, buf_k=None, buf_u=None, buf_g=None,
                 n=None) -> None:
    """Write an oracle-made state into GPU buffers (rounded to fp32)."""
    def put(dst: torch.Tensor, x):
        dst.copy_(torch.from_numpy(np.ascontiguousarray(np.asarray(x, np.float32).reshape(dst.shape))))
    st.codes.copy_(torch.from_numpy(pack_codes(enc.codes, dims.bits)).reshape(st.codes.shape))
    put(st.row_scale, enc.s)
    put(st.col_scale, enc.c)
    if dims.n_comp:
        put(st.comp_k, enc.comp_k)
        put(st.comp_u, enc.comp_u)
        st.ent_g[:, :dims.n_comp] = 0.0  # compensators sit at window position 0
    if buf_k is not None:
        put(st.buf_k, buf_key_rows(np.asarray(buf_k, np.float32).reshape(st.buf_k.shape), dims))
        put(st.buf_u, buf_u)
        put(st.buf_g, buf_g)
        st.buf_len.copy_(torch.from_numpy(np.asarray(n, np.int32)))
    else:
        st.buf_len.zero_()


def heads_of(seqs: Sequence[int], H: int) -> np.ndarray:
    return (np.asarray(seqs)[:, None] * H + np.arange(H)[None, :]).reshape(-1)


def overwrite_heads(st: lqk.State, dims: lqk.Dims, gpu_heads, enc: lq.Encoded) -> None:
    """Replace the window-start state of some heads by an oracle encoding (fp32)."""
    idx = torch.as_tensor(np.asarray(gpu_heads), device="cuda", dtype=torch.long)
    dev = lambda x, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)
    st.codes[idx] = dev(pack_codes(enc.codes, dims.bits), torch.int8)
    st.row_scale[idx] = dev(np.asarray(enc.s, np.float32))
    st.col_scale[idx] = dev(np.asarray(enc.c, np.float32))
    if dims.n_comp:
        st.ent_k[idx, :dims.n_comp] = dev(np.asarray(enc.comp_k, np.float32))
        st.ent_u[idx, :dims.n_comp] = dev(np.asarray(enc.comp_u, np.float32))


def run_gpu(wl: wk.Workload, steps: int, check_seqs: Sequence[int], bits=None, chunk: int = 16,
            force=None):
    """HIP path over the full batch; returns outputs of check_seqs [steps][S][H][d].

    force: an oracle result of run_oracle(..., record=True) on check_seqs. The
    checked heads then start every window from the oracle's encoding (teacher
    forcing): after the GPU closes a window, those heads are overwritten with
    the oracle's Enc of the same window, so each window's outputs test the
    kernels' arithmetic without the history of earlier rounding decisions."""
    dims = runner.dims_for(wl, bits)
    dec = runner.Decoder(dims, wk.window_lengths(wl), wk.window_offsets(wl))
    S0 = wk.initial_states(wl, range(wl.batch))
    dec.encode(runner.states_to_device(S0))
    del S0
    gheads = heads_of(check_seqs, wl.heads)
    closes = {}
    if force is not None:
        overwrite_heads(dec.state, dims, gheads, force["enc0"])
        closes = {ev.step: ev for ev in force["closes"]}
    stream = wk.TokenStream(wl)
    sel = torch.as_tensor(np.asarray(check_seqs), device="cuda", dtype=torch.long)
    outs = torch.empty((steps, len(check_seqs), wl.heads, wl.d_v), dtype=torch.float32, device="cuda")
    for c0 in range(0, steps, chunk):
        n = min(chunk, steps - c0)
        dev = runner.upload_tokens(stream.next(n), wl.act_bf16)
        for i in range(n):
            t = c0 + i
            o = dec.step(dev["q"][i], dev["k"][i], dev["v"][i], dev["g"][i], dev["beta"][i])
            outs[t] = o.view(wl.batch, wl.heads, wl.d_v).index_select(0, sel)
            if t in closes:
                overwrite_heads(dec.state, dims, gheads[closes[t].heads], closes[t].enc)
        del dev
    torch.cuda.synchronize()
    err = int(dec.state.err.item())
    return outs.cpu().numpy(), dec, err


def run_oracle(wl: wk.Workload, steps: int, seqs: Sequence[int], bits=None, record=False,
               rounding_noise: float = 0.0, noise_seed: int = 1):
    """fp64 plain definition on the listed sequences (same per-sequence inputs)."""
    S0 = wk.initial_states(wl, seqs).reshape(-1, wl.d_k, wl.d_v).astype(np.float64)
    toks = flat_steps(wk.TokenStream(wl, seqs).next(steps))
    H = wl.heads
    win_len = np.repeat(wk.window_lengths(wl)[list(seqs)], H)
    win_off = np.repeat(wk.window_offsets(wl)[list(seqs)], H)
    res = lq.run_dense(S0, toks, win_len, win_off, r=wl.n_comp, T=wl.power_iters,
                       bits=wl.bits if bits is None else bits, smoothing=wl.smoothing, record=record,
                       rounding_noise=rounding_noise, noise_seed=noise_seed, warm_start=wl.warm_start)
    res["o"] = res["o"].reshape(steps, len(seqs), H, wl.d_v)
    return res


def g1_check(R_gpu_math: np.ndarray, host: Dict[str, np.ndarray], bits: int, smoothing: bool,
             heads=None):
    """Staged code gate: oracle E3-E4 in fp64 on the GPU's own fp32 residual."""
    idx = slice(None) if heads is None else heads
    s, c, C = lq.smooth_quantize(R_gpu_math.astype(np.float64), bits, smoothing)
    Cg = host["C"][idx]
    same = float(np.mean(Cg == C))
    max_diff = int(np.max(np.abs(Cg - C)))
    s_gpu = host["row_scale"][idx]
    c_gpu = host["col_scale"][idx]
    s_exact = bool(np.array_equal(s_gpu, s.astype(np.float32)))
    c_ref = c.astype(np.float32)
    ulp = np.spacing(np.maximum(np.abs(c_ref), np.float32(1e-38)).astype(np.float32))
    c_ulps = float(np.max(np.abs(c_gpu.astype(np.float64) - c_ref.astype(np.float64)) / ulp))
    return dict(same=same, max_diff=max_diff, s_exact=s_exact, c_ulps=c_ulps)


def download_heads(st: lqk.State, dims: lqk.Dims, heads) -> Dict[str, np.ndarray]:
    """download_state restricted to the listed heads (gathered on the device)."""
    torch.cuda.synchronize()
    idx = torch.as_tensor(np.asarray(heads), device="cuda", dtype=torch.long)
    out = {n: getattr(st, n).index_select(0, idx).cpu().numpy() for n in lqk.STATE_FIELDS if n != "err"}
    out["C"] = unpack_codes(out["codes"], dims.bits, dims.d)
    r = dims.n_comp
    out["comp_k"], out["comp_u"], out["comp_g"] = out["ent_k"][:, :r], out["ent_u"][:, :r], out["ent_g"][:, :r]
    out["buf_k"], out["buf_u"], out["buf_g"] = buf_keys_f32(out["ent_k"], dims), out["ent_u"][:, r:], out["ent_g"][:, r:]
    return out


def run_gpu_closes(wl: wk.Workload, steps: int, check_seqs: Sequence[int], bits=None, on_close=None,
                   chunk: int = 16):
    """Free-running HIP path over the full batch, like run_gpu, with a hook at
    every window close: on_close(t, local, pre, post, R) gets the step, the
    indices (into the checked heads) of the checked heads that close, their
    state just before and just after the close, and the residual the close
    quantized (host arrays, checked heads only; R in the math layout).
    Returns (outputs of check_seqs [steps][S][H][d], Decoder, error word, the
    checked heads' state after the initial encode)."""
    dims = runner.dims_for(wl, bits)
    win_len, win_off = wk.window_lengths(wl), wk.window_offsets(wl)
    dec = runner.Decoder(dims, win_len, win_off)
    S0 = wk.initial_states(wl, range(wl.batch))
    dec.encode(runner.states_to_device(S0))
    del S0
    gheads = heads_of(check_seqs, wl.heads)
    start = download_heads(dec.state, dims, gheads)
    dbg = torch.zeros((wl.batch * wl.heads, wl.d_v, wl.d_k), dtype=torch.float32, device="cuda")
    seq_of = np.asarray(check_seqs)
    stream = wk.TokenStream(wl)
    sel = torch.as_tensor(seq_of, device="cuda", dtype=torch.long)
    outs = torch.empty((steps, len(check_seqs), wl.heads, wl.d_v), dtype=torch.float32, device="cuda")
    for c0 in range(0, steps, chunk):
        n = min(chunk, steps - c0)
        dev = runner.upload_tokens(stream.next(n), wl.act_bf16)
        for i in range(n):
            t = c0 + i
            o = dec.step(dev["q"][i], dev["k"][i], dev["v"][i], dev["g"][i], dev["beta"][i], close=False)
            outs[t] = o.view(wl.batch, wl.heads, wl.d_v).index_select(0, sel)
            due = (win_off[seq_of].astype(np.int64) + t + 1) % win_len[seq_of] == 0
            if dec.closes_at(t) and on_close is not None and np.any(due):
                local = np.nonzero(np.repeat(due, wl.heads))[0]
                pre = download_heads(dec.state, dims, gheads[local])
                dec.close_due(t, dbg)
                post = download_heads(dec.state, dims, gheads[local])
                idx = torch.as_tensor(gheads[local], device="cuda", dtype=torch.long)
                on_close(t, local, pre, post, T(dbg.index_select(0, idx).cpu().numpy()))
            else:
                dec.close_due(t)
        del dev
    torch.cuda.synchronize()
    err = int(dec.state.err.item())
    return outs.cpu().numpy(), dec, err, start

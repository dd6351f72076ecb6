#!/usr/bin/env python3
"""Decode throughput of LeapQuant on one MI355X: the int8 decode step plus its
window closes, against the FP32-state baseline on identical inputs.

Default workload: Qwen-style GDN decode, 64 sequences x 32 heads,
d_k = d_v = 128, window W = 16, r = 4 compensators, int8 residual with
per-key-row smoothing and per-value-column scales, bf16 q/k/v (synthetic,
seeded). L = 8 independent state sets, one per linear-attention layer of a
model, are advanced in turn, so each launch reads its state from HBM and not
from the 256 MB Infinity Cache.

One step = one decode token for every head of every layer, plus the window
closes that fall on that token. The timed region replays HIP graphs: the
decode launches between two close points form one graph, the closes due at a
point another; HIP events on the replay stream bracket every graph, which
gives the average duration of each kernel. The whole region is bracketed by
device synchronisation on both sides.

Prints one JSON line. The roofline object describes the decode-step kernel:
achieved = algorithmic bytes per launch / average launch duration; traffic =
HBM bytes per launch read by the FETCH_SIZE and WRITE_SIZE counters (scaled by
their reading on a plain copy of known size), taken from the committed counter
profile while the kernel sources are unchanged since, else null.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--layers", type=int, default=8)
    p.add_argument("--workload", default="qwen_gdn")
    p.add_argument("--bits", type=int, default=None)
    p.add_argument("--power-iters", type=int, default=None, help="power iterations per compensator")
    p.add_argument("--warm-start", action="store_true",
                   help="start each close's power method from the closing window's compensators")
    p.add_argument("--no-fp32", action="store_true", help="skip the FP32-state baseline")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    p.add_argument("--cpu-sample", default="32x256", help="oracle sample: sequences x steps")
    p.add_argument("--prefill-tokens", type=int, default=256,
                   help="prompt length of the prefill-handoff leg (0: skip)")
    p.add_argument("--no-snapshot", action="store_true", help="skip timing snapshot/restore")
    p.add_argument("--no-overlap", action="store_true",
                   help="skip the schedule with window closes overlapping other layers' decodes")
    p.add_argument("--no-stream-reference", action="store_true",
                   help="skip timing plain library streaming of the same bytes")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device copy three times (the reference dispatch "
                        "for scaling hardware byte counters), then exit")
    return p.parse_args()


def copy_calibration():
    """A plain copy of known size: a counter profile of these dispatches gives
    the factor between what the HBM byte counters read and the bytes moved."""
    import torch
    n = 256 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_dispatch": n, "bytes_written_per_dispatch": n,
                                           "dispatches": 3}}), flush=True)


def stream_reference(nbytes, layers=8, reps=20):
    """A plain device copy moving the decode launch's byte count (half read, half
    written) through the runtime's copy path, one buffer pair per layer so that
    the last-level cache does not hold them, launched back to back: a reference
    for the decode kernel's HBM fraction on this device, not part of the step."""
    import torch
    n = (nbytes // 2) // 4  # fp32 elements copied per launch
    src = [torch.ones(n, dtype=torch.float32, device="cuda") for _ in range(layers)]
    dst = [torch.empty_like(x) for x in src]
    for d, x in zip(dst, src):
        d.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for d, x in zip(dst, src):
            d.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * layers)
    moved = 2 * n * 4
    return {"kind": "device copy", "bytes_per_launch": moved, "us_per_launch": round(us, 2),
            "gbs": round(moved / (us * 1e-6) / 1e9, 1)}


def schedule(win_len, win_off, total):
    """Per step: list of sequences whose window closes after it; per step and
    sequence the number of tokens already buffered (n)."""
    import numpy as np
    B = len(win_len)
    n = np.zeros(B, np.int64)
    closes, ns = [], []
    for t in range(total):
        ns.append(n.copy())
        n += 1
        due = np.nonzero((win_off.astype(np.int64) + t + 1) % win_len == 0)[0]
        closes.append(due)
        n[due] = 0
    return closes, ns


def segments(closes, t0, t1):
    """Split steps [t0, t1) after every step with a close."""
    segs, start = [], t0
    for t in range(t0, t1):
        if len(closes[t]) or t == t1 - 1:
            segs.append((start, t + 1))
            start = t + 1
    return segs


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_step_kernel_qwen_gdn_traffic.md")
KERNEL_SOURCES = ("decode_step.hip", "lq_common.h", "lq_launch.h")


def measured_traffic(wl, bits):
    """HBM bytes per decode launch from the committed counter profile (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy's reading), or None when the profile does not
    cover this workload or the kernel sources changed since it was taken."""
    import hashlib
    if wl.name != "qwen_gdn" or bits != 8 or not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for ln in open(TRAFFIC_PROFILE):
        if ":" in ln and ln.split(":")[0] in ("traffic_bytes_per_launch", "source_sha256"):
            k, v = ln.split(":", 1)
            fields[k] = v.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "linear_attention_recurrent_kda_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def run_gpu(args, wl, bits):
    import numpy as np
    import torch

    from linear_attention_recurrent_kda_amd import bytes_model as bm
    from linear_attention_recurrent_kda_amd import leapquant as lqk
    from linear_attention_recurrent_kda_amd import runner
    from linear_attention_recurrent_kda_amd import workloads as wk

    torch.cuda.set_device(0)
    L, K, Wu = args.layers, args.steps, args.warmup
    total = Wu + K
    dims = runner.dims_for(wl, bits)
    BH, D = wl.batch * wl.heads, wl.d_k
    win_len, win_off = wk.window_lengths(wl), wk.window_offsets(wl)
    closes, ns = schedule(win_len, win_off, total)

    # inputs resident in HBM before anything is timed
    S_init = runner.states_to_device(wk.initial_states(wl, range(wl.batch)))
    toks = [wk.device_tokens(wl, total, seed=l) for l in range(L)]
    states = [lqk.State(dims) for _ in range(L)]
    for st in states:
        lqk.encode(dims, S_init, st)
    outs = [torch.empty((BH, D), dtype=torch.float32, device="cuda") for _ in range(L)]
    close_ids = {}  # distinct close lists, uploaded once

    def ids_for(t):
        key = tuple(int(b) for b in closes[t])
        if key not in close_ids:
            close_ids[key] = torch.tensor(key, dtype=torch.int32, device="cuda")
        return close_ids[key]

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    def dec_graph(a, b):
        def body():
            for t in range(a, b):
                for l in range(L):
                    x = toks[l]
                    lqk.decode_step(dims, states[l], x["q"][t], x["k"][t], x["v"][t], x["g"][t],
                                    x["beta"][t], outs[l])
        return capture(body)

    def close_graph(t):
        ids = ids_for(t)
        all_seqs = len(closes[t]) == wl.batch

        def body():
            for l in range(L):
                if all_seqs:
                    lqk.window_close(dims, states[l], None, 0)
                else:
                    lqk.window_close(dims, states[l], ids, len(closes[t]))
        return capture(body)

    torch.cuda.synchronize()
    # capture: one decode graph per segment, one close graph per distinct close list
    plan = []
    cgraphs = {}
    for (a, b) in segments(closes, 0, total):
        g_dec = dec_graph(a, b)
        key = tuple(int(x) for x in closes[b - 1])
        if key and key not in cgraphs:
            cgraphs[key] = close_graph(b - 1)
        plan.append((a, b, g_dec, cgraphs.get(key) if key else None))
    torch.cuda.synchronize()
    # capture ran nothing; start from freshly encoded states
    for st in states:
        lqk.encode(dims, S_init, st)
    torch.cuda.synchronize()

    def replay(lo, hi, timed):
        evs = []
        for (a, b, g_dec, g_close) in plan:
            if a < lo or a >= hi:
                continue
            if timed:
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record()
            g_dec.replay()
            if timed:
                e1.record()
            if g_close is not None:
                g_close.replay()
            if timed:
                e2.record()
                evs.append((a, b, e0, e1, e2, g_close is not None))
        return evs

    replay(0, Wu, timed=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs = replay(Wu, total, timed=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    err = int(sum(int(st.err.item()) for st in states))
    assert err == 0, f"device error word {err}"

    # per-kernel averages from the events and algorithmic bytes from the schedule
    dec_us = close_us = 0.0
    n_dec = n_close = 0
    dec_bytes = close_bytes = 0
    H = wl.heads
    for (a, b, e0, e1, e2, has_close) in evs:
        dec_us += e0.elapsed_time(e1) * 1e3
        n_dec += (b - a) * L
        for t in range(a, b):
            dec_bytes += L * H * sum(bm.step_bytes(D, wl.n_comp, dims.bits, wl.kda, wl.act_bf16, int(n))
                                     for n in ns[t])
        if has_close:
            close_us += e1.elapsed_time(e2) * 1e3
            n_close += L
            t = b - 1
            close_bytes += L * H * sum(bm.close_bytes(D, wl.n_comp, dims.bits, wl.kda, wl.act_bf16,
                                                      int(ns[t][s]) + 1) for s in closes[t])
    res = dict(wall=wall, dec_us=dec_us / max(n_dec, 1), close_us=close_us / max(n_close, 1),
               n_dec=n_dec, n_close=n_close, dec_bytes=dec_bytes, close_bytes=close_bytes,
               dec_gbs=dec_bytes / (dec_us * 1e-6) / 1e9 if dec_us else 0.0,
               head_tokens=K * L * BH, state_mb=states[0].nbytes() / 1e6)

    # The same steps with the window closes overlapped: runner.capture_tokens puts
    # the close of layer l on a side stream as soon as layer l's decode is done;
    # only layer l's next decode waits for it (bit-identical results).
    if not args.no_overlap:
        del states
        decs = [runner.Decoder(dims, win_len, win_off) for _ in range(L)]
        for d in decs:
            d.encode(S_init)
        g_warm = runner.capture_tokens(decs, toks, outs, 0, Wu, overlap=True)
        g_timed = runner.capture_tokens(decs, toks, outs, Wu, total, overlap=True)
        for d in decs:
            d.encode(S_init)
        torch.cuda.synchronize()
        g_warm.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g_timed.replay()
        torch.cuda.synchronize()
        res["overlap_wall"] = time.perf_counter() - t0
        assert sum(int(d.state.err.item()) for d in decs) == 0
        del decs, g_warm, g_timed
        states = None

    # FP32-state baseline on identical inputs and the same protocol
    if not args.no_fp32:
        states = None
        lq_last = torch.stack([o.clone() for o in outs])  # LeapQuant outputs of the last step
        Sf = [S_init.clone() for _ in range(L)]

        def fp_graph(a, b):
            def body():
                for t in range(a, b):
                    for l in range(L):
                        x = toks[l]
                        lqk.fp32_baseline_step(dims, Sf[l], x["q"][t], x["k"][t], x["v"][t], x["g"][t],
                                               x["beta"][t], outs[l])
            return capture(body)
        fplan = [(a, b, fp_graph(a, b)) for (a, b) in segments(closes, 0, total)]
        for l in range(L):
            Sf[l].copy_(S_init)
        for (a, b, g) in fplan:
            if a < Wu:
                g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fevs = []
        for (a, b, g) in fplan:
            if a >= Wu:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                g.replay()
                e1.record()
                fevs.append((a, b, e0, e1))
        torch.cuda.synchronize()
        fwall = time.perf_counter() - t0
        fus = sum(e0.elapsed_time(e1) * 1e3 for (_, _, e0, e1) in fevs)
        fn = sum((b - a) * L for (a, b, _, _) in fevs)
        fbytes = fn * BH * bm.fp32_step_bytes(D, wl.kda, wl.act_bf16)
        res.update(fp32_wall=fwall, fp32_us=fus / fn, fp32_gbs=fbytes / (fus * 1e-6) / 1e9)
        # both runs saw the same inputs: the last step's outputs against the exact fp32 recurrence
        fp_last = torch.stack(outs)
        res["quality_rel_l2"] = float(torch.linalg.vector_norm(lq_last - fp_last) /
                                      torch.linalg.vector_norm(fp_last))
    return res


FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X, fp32 vector (counts packed dual-rate FP32)
FP32_MFMA_PEAK_TFLOPS = 157.3    # MI355X, dense fp32 matrix


def run_prefill(wl, bits, n_tokens):
    """Prefill handoff: the exact recurrence over a prompt of n_tokens (fp32 state
    on chip), then the encode into LeapQuant form. Algorithmic work: 7 d^2 flops
    per head-token (decay, the two column sums S'^T k and S'^T q, the rank-one
    update). At d = 128 the prompt runs in chunks on the matrix cores (bound:
    fp32 MFMA); below that, token by token on the vector ALU."""
    import torch

    from linear_attention_recurrent_kda_amd import leapquant as lqk
    from linear_attention_recurrent_kda_amd import runner
    from linear_attention_recurrent_kda_amd import workloads as wk

    dims = runner.dims_for(wl, bits)
    N, d = wl.batch * wl.heads, wl.d_k
    S0 = runner.states_to_device(wk.initial_states(wl, range(wl.batch)))
    x = wk.device_tokens(wl, n_tokens, seed=100)
    o = torch.empty((n_tokens, N, d), dtype=torch.float32, device="cuda")
    S = torch.empty_like(S0)
    st = lqk.State(dims)
    runs = []
    for rep in range(3):
        S.copy_(S0)
        torch.cuda.synchronize()
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record()
        lqk.prefill(dims, S, x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        e1.record()
        lqk.encode(dims, S, st)
        e2.record()
        torch.cuda.synchronize()
        runs.append((e0.elapsed_time(e1) * 1e3, e1.elapsed_time(e2) * 1e3))
    pre_us, enc_us = min(runs)
    flops = 7.0 * d * d * N * n_tokens
    tflops = flops / (pre_us * 1e-6) / 1e12
    mfma = d == 128
    bound, peak = ("mfma", FP32_MFMA_PEAK_TFLOPS) if mfma else ("alu", FP32_VECTOR_PEAK_TFLOPS)
    return {"prompt_tokens": n_tokens, "head_tokens_per_s": round(N * n_tokens / (pre_us * 1e-6), 1),
            "prefill_us": round(pre_us, 1), "encode_us": round(enc_us, 1),
            "roofline": {"bound": bound, "achieved": round(tflops, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(tflops / peak, 4)}}


def outlier_report(wl, bits, n_seq=8):
    """Outlier-to-median ratio max|X| / median|X| per head, median and max over the
    heads of the first n_seq sequences: the initial state S, the GPU encode's residual R (after
    the compensators) and R / s (after key-row smoothing). Reported in kind with the
    pages' example, not a target."""
    import numpy as np
    import torch

    from linear_attention_recurrent_kda_amd import leapquant as lqk
    from linear_attention_recurrent_kda_amd import runner
    from linear_attention_recurrent_kda_amd import workloads as wk

    small = wl.replace(batch=n_seq)
    dims = runner.dims_for(small, bits)
    N, d = small.batch * small.heads, small.d_k
    S = runner.states_to_device(wk.initial_states(small, range(n_seq)))
    st = lqk.State(dims)
    R = torch.empty((N, d, d), dtype=torch.float32, device="cuda")
    lqk.encode(dims, S, st, R)
    torch.cuda.synchronize()
    # both stored transposed ([d_v][d_k]); the ratio does not depend on orientation
    s_rows = st.row_scale.cpu().numpy()  # per key channel
    Rh = R.cpu().numpy()
    def ratio(X):
        r = np.array([np.max(np.abs(x)) / np.median(np.abs(x)) for x in X])
        return {"median": round(float(np.median(r)), 1), "max": round(float(r.max()), 1)}
    return {"heads": N, "state": ratio(S.cpu().numpy()), "after_compensators": ratio(Rh),
            "after_smoothing": ratio(Rh / s_rows[:, None, :])}


def run_snapshot(wl, bits):
    """Prefix-cache snapshot and restore of every sequence at a window boundary.
    HBM-bound copies: one record per head read and written once each way."""
    import torch

    from linear_attention_recurrent_kda_amd import leapquant as lqk
    from linear_attention_recurrent_kda_amd import runner
    from linear_attention_recurrent_kda_amd import workloads as wk

    dims = runner.dims_for(wl, bits)
    N, d = wl.batch * wl.heads, wl.d_k
    st = lqk.State(dims)
    lqk.encode(dims, runner.states_to_device(wk.initial_states(wl, range(wl.batch))), st)
    rec = lqk.snapshot_bytes(dims)
    snap = torch.empty((wl.batch, wl.heads, rec), dtype=torch.uint8, device="cuda")
    best = {}
    for name, fn in (("snapshot", lqk.snapshot), ("restore", lqk.restore)):
        fn(dims, st, snap)  # warm-up
        torch.cuda.synchronize()
        times = []
        reps = 20  # back to back, so that host call overhead does not idle the GPU
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn(dims, st, snap)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / reps)
        best[name] = min(times)
    assert int(st.err.item()) == 0
    moved = 2.0 * rec * N  # each record read once and written once
    gbs = moved / (best["snapshot"] * 1e-6) / 1e9
    return {"record_bytes_per_head": rec, "fp32_state_bytes_per_head": 4 * d * d,
            "heads": N, "snapshot_us": round(best["snapshot"], 1), "restore_us": round(best["restore"], 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def cpu_baseline(wl, bits, sample):
    """The fp64 oracle (plain definition) on a bounded sample of the same workload."""
    import numpy as np

    from linear_attention_recurrent_kda_amd import workloads as wk
    from oracle import leapquant_oracle as lq

    n_seq, n_steps = (int(x) for x in sample.split("x"))
    seqs = list(range(n_seq))
    raw = wk.TokenStream(wl, seqs).next(n_steps)
    toks = [{k: raw[k][t].reshape((-1,) + raw[k].shape[3:]).astype(np.float64)
             for k in ("q", "k", "v", "g", "beta")} for t in range(n_steps)]
    S0 = wk.initial_states(wl, seqs).reshape(-1, wl.d_k, wl.d_v).astype(np.float64)
    N = S0.shape[0]
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    t0 = time.perf_counter()
    lq.run_dense(S0, toks, np.repeat(wk.window_lengths(wl)[seqs], wl.heads),
                 np.repeat(wk.window_offsets(wl)[seqs], wl.heads), r=wl.n_comp, T=wl.power_iters,
                 bits=bits, smoothing=wl.smoothing)
    dt = time.perf_counter() - t0
    return dict(value=N * n_steps / dt, unit="head-tokens/s", cores=threads, kind="oracle",
                sample=f"{n_seq} sequences x {wl.heads} heads x {n_steps} tokens of the same workload "
                       f"(initial encode + {n_steps // wl.window} window closes), numpy fp64, "
                       f"{dt:.1f} s; BLAS threads {threads}, {len(os.sched_getaffinity(0))} cores visible")


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the decode path has no cross-GPU exchange (heads and "
              f"sequences shard with no communication), so --gpus {args.gpus} is not run.",
              file=sys.stderr)
        sys.exit(2)
    from linear_attention_recurrent_kda_amd import workloads as wk

    wl = wk.WORKLOADS[args.workload]
    if args.power_iters is not None:
        wl = wl.replace(power_iters=args.power_iters)
    if args.warm_start:
        wl = wl.replace(warm_start=True)
    bits = wl.bits if args.bits is None else args.bits
    r = run_gpu(args, wl, bits)
    value = r["head_tokens"] / r["wall"]
    line = {
        "metric": "decode head-tokens/s + achieved HBM GB/s (int8 LeapQuant vs FP32 state)",
        "value": round(value, 1),
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall"] * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {'KDA' if wl.kda else 'GDN'} decode, {wl.batch} sequences x "
                        f"{wl.heads} heads, d_k=d_v={wl.d_k}, W={wl.window if not wl.mixed_window else '16/32'}, "
                        f"r={wl.n_comp}, int{bits} state, {'bf16' if wl.act_bf16 else 'fp32'} q/k/v; "
                        f"{args.layers} layers' state sets advanced per step",
            "batch": wl.batch, "heads": wl.heads, "d_k": wl.d_k, "d_v": wl.d_v, "window": wl.window,
            "n_comp": wl.n_comp, "state_bits": bits, "layers": args.layers,
            "power_iters": wl.power_iters, "warm_start": wl.warm_start,
            "state_mb_per_layer": round(r["state_mb"], 1),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(r["dec_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["dec_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(wl, bits),
            "kernel": "decode_step_kernel",
            "avg_launch_us": round(r["dec_us"], 3),
            "bytes_per_launch": round(r["dec_bytes"] / max(r["n_dec"], 1)),
        },
        "window_close": {"avg_launch_us": round(r["close_us"], 3), "launches": r["n_close"],
                         "bytes_per_launch": round(r["close_bytes"] / max(r["n_close"], 1))},
        "hbm_gbs_all_in": round((r["dec_bytes"] + r["close_bytes"]) / r["wall"] / 1e9, 1),
    }
    if "overlap_wall" in r:
        line["overlapped_schedule"] = {
            "value": round(r["head_tokens"] / r["overlap_wall"], 1), "unit": "head-tokens/s",
            "ms_per_step": round(r["overlap_wall"] * 1e3 / args.steps, 4),
            "note": "the same steps, each layer's window close on a side stream beside the other "
                    "layers' decodes (bit-identical results); value above is the in-order schedule"}
    if "fp32_us" in r:
        fval = r["head_tokens"] / r["fp32_wall"]
        line["fp32_baseline"] = {"value": round(fval, 1), "unit": "head-tokens/s",
                                 "avg_launch_us": round(r["fp32_us"], 3),
                                 "achieved_gbs": round(r["fp32_gbs"], 1)}
        line["speedup_vs_fp32"] = round(value / fval, 3)
        line["fp32_baseline"]["leapquant_output_rel_l2"] = round(r["quality_rel_l2"], 6)
    if args.prefill_tokens > 0:
        line["prefill_handoff"] = run_prefill(wl, bits, args.prefill_tokens)
    if not args.no_snapshot:
        line["snapshot"] = run_snapshot(wl, bits)
    line["outlier_ratio"] = outlier_report(wl, bits)
    if not args.no_stream_reference:
        line["stream_reference"] = stream_reference(r["dec_bytes"] // max(r["n_dec"], 1), args.layers)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, bits, args.cpu_sample)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

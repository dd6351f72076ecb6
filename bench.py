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
closes that fall on that token. The timed region is exactly the --steps steps
after the --warmup steps, with every close due in it: HIP graphs are captured
per run of decode steps between two close points (split at the warm-up
boundary too), and per distinct close list; HIP events on the replay stream
bracket every graph, which gives the average duration of each kernel. The
timed loop runs five times from the same post-warm-up state (restored, untimed,
before each repeat) and the median is reported; device synchronisation
brackets each repeat. The event totals must lie inside the wall-clock region
and no byte rate may exceed the HBM peak (asserted).

Prints one JSON line. The roofline object describes the decode-step kernel over
the timed steps (their window positions are listed): achieved = algorithmic
bytes per launch / average launch duration; whole_windows gives the same over
one full period of the close schedule from a fresh encode. traffic = HBM bytes
per launch read by the FETCH_SIZE and WRITE_SIZE counters (scaled by their
reading on a plain copy of known size), taken from the committed counter
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
    p.add_argument("--cpu-sample", default="16x256", help="oracle sample: sequences x steps")
    p.add_argument("--prefill-tokens", type=int, default=256,
                   help="prompt length of the prefill-handoff leg (0: skip)")
    p.add_argument("--no-snapshot", action="store_true", help="skip timing snapshot/restore")
    p.add_argument("--no-fuse", action="store_true",
                   help="take a window's last token with a decode launch and then close, instead of in one launch")
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
    """Split steps [t0, t1) after every step with a close (and at t1): every
    close due at a step in [t0, t1) belongs to the segment that ends with it."""
    segs, start = [], t0
    for t in range(t0, t1):
        if len(closes[t]) or t == t1 - 1:
            segs.append((start, t + 1))
            start = t + 1
    return segs


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_step_kernel_qwen_gdn_traffic.md")
KERNEL_SOURCES = ("decode_step.hip", "lq_common.h", "lq_launch.h")
REPEATS = 5  # timed loop repeats; the median is reported


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


def _median_run(runs):
    """The run with the median wall time of an odd number of runs."""
    return sorted(runs, key=lambda r: r["wall"])[len(runs) // 2]


def positions_text(ns_list):
    """Window positions (tokens already buffered) covered by the timed steps:
    {position: sequence-steps at that position / batch}, i.e. the number of
    timed steps at each position when every sequence shares its window."""
    import numpy as np
    allpos = np.concatenate(ns_list) if ns_list else np.zeros(0, np.int64)
    vals, counts = np.unique(allpos, return_counts=True)
    B = len(ns_list[0]) if ns_list else 1
    return {int(v): round(float(c) / B, 2) for v, c in zip(vals, counts)}


class Graphs:
    """HIP graphs of the decode schedule over L layer state sets: one graph per
    run of decode steps between two close points (every layer's launch for
    each step), one graph per distinct close list (every layer's close). With
    fuse, a step after which every sequence closes, all at the same window
    position, is one launch per layer (leapquant_decode_close_at: the token's
    step inside the close) in a graph of its own, and the decode graph before
    it ends one step earlier."""

    def __init__(self, dims, states, toks, outs, closes, lqk, torch, kind="leapquant", ns=None, fuse=True):
        self.dims, self.states, self.toks, self.outs = dims, states, toks, outs
        self.closes, self.lqk, self.torch, self.kind = closes, lqk, torch, kind
        self.ns = ns  # per step, the tokens each sequence holds (None: the kernel reads them)
        self.fuse = fuse and kind == "leapquant" and ns is not None
        self._ids, self._cg, self._fg = {}, {}, {}

    def fused_at(self, t):
        """The window position of step t when that step is taken inside the
        close (every sequence closes after it, all at one position), else -1."""
        if not self.fuse or len(self.closes[t]) != self.dims.batch:
            return -1
        n = self.ns[t]
        return int(n[0]) if (n == n[0]).all() else -1

    def _capture(self, fn):
        g = self.torch.cuda.CUDAGraph()
        with self.torch.cuda.graph(g):
            fn()
        return g

    def decode(self, a, b):
        """The decode graph of steps [a, b) (None when empty)."""
        if b <= a:
            return None
        lqk, dims = self.lqk, self.dims

        def body():
            for t in range(a, b):
                # every sequence at the same window position: the kernel is told it
                n = int(self.ns[t][0]) if self.ns is not None and (self.ns[t] == self.ns[t][0]).all() else -1
                for l, st in enumerate(self.states):
                    x = self.toks[l]
                    if self.kind == "leapquant" and n >= 0:
                        lqk.decode_step_at(dims, st, n, x["q"][t], x["k"][t], x["v"][t], x["g"][t], x["beta"][t],
                                           self.outs[l])
                    elif self.kind == "leapquant":
                        lqk.decode_step(dims, st, x["q"][t], x["k"][t], x["v"][t], x["g"][t], x["beta"][t],
                                        self.outs[l])
                    else:
                        lqk.fp32_baseline_step(dims, st, x["q"][t], x["k"][t], x["v"][t], x["g"][t],
                                               x["beta"][t], self.outs[l])
        return self._capture(body)

    def close(self, t):
        """The close graph of the sequences due after step t (None when none or
        FP32); with fusion, step t itself inside the close."""
        if self.kind != "leapquant" or not len(self.closes[t]):
            return None
        n = self.fused_at(t)
        if n >= 0:
            if t not in self._fg:
                lqk, dims = self.lqk, self.dims

                def fused():
                    for l, st in enumerate(self.states):
                        x = self.toks[l]
                        lqk.decode_close_at(dims, st, n, x["q"][t], x["k"][t], x["v"][t], x["g"][t],
                                            x["beta"][t], self.outs[l])
                self._fg[t] = self._capture(fused)
            return self._fg[t]
        key = tuple(int(b) for b in self.closes[t])
        if key not in self._cg:
            if key not in self._ids:
                self._ids[key] = self.torch.tensor(key, dtype=self.torch.int32, device="cuda")
            ids, lqk, dims = self._ids[key], self.lqk, self.dims
            every = len(key) == dims.batch

            def body():
                for st in self.states:
                    if every:
                        lqk.window_close(dims, st, None, 0)
                    else:
                        lqk.window_close(dims, st, ids, len(key))
            self._cg[key] = self._capture(body)
        return self._cg[key]

    def plan(self, t0, t1):
        """[(a, b, decode graph or None, close graph or None, fused)] covering
        steps [t0, t1); fused: step b - 1 is taken inside the close graph."""
        out = []
        for (a, b) in segments(self.closes, t0, t1):
            f = self.fused_at(b - 1) >= 0
            out.append((a, b, self.decode(a, b - 1 if f else b), self.close(b - 1), f))
        return out


def replay(plan, torch, timed):
    """Replay a plan in order; with timed, HIP events (torch's, on the replay
    stream) bracket each decode graph and each close graph."""
    evs = []
    for (a, b, g_dec, g_close, fused) in plan:
        if timed:
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record()
        if g_dec is not None:
            g_dec.replay()
        if timed:
            e1.record()
        if g_close is not None:
            g_close.replay()
        if timed:
            e2.record()
            evs.append((a, b, e0, e1, e2, g_close is not None, fused))
    return evs


def timed_repeats(plan, tensors, torch, check_err=None, repeats=REPEATS):
    """Replay the timed plan `repeats` times, each from the same starting state
    (the tensors are restored from a copy taken now, untimed); device
    synchronisation brackets each timed replay. Returns the median run:
    wall seconds and per-segment event times (µs)."""
    saved = [x.clone() for x in tensors]
    runs = []
    for _ in range(repeats):
        for x, s in zip(tensors, saved):
            x.copy_(s)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs = replay(plan, torch, timed=True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if check_err is not None:
            check_err()
        seg = [(a, b, e0.elapsed_time(e1) * 1e3, e1.elapsed_time(e2) * 1e3 if hc else 0.0, hc, fu)
               for (a, b, e0, e1, e2, hc, fu) in evs]
        runs.append(dict(wall=wall, seg=seg))
    del saved
    return _median_run(runs), sorted(r["wall"] for r in runs)


def run_gpu(args, wl, bits):
    import math

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
    BH, D, H = wl.batch * wl.heads, wl.d_k, wl.heads
    win_len, win_off = wk.window_lengths(wl), wk.window_offsets(wl)
    period = int(np.lcm.reduce(win_len))  # the close schedule repeats with this period
    n_tok = max(total, 2 * period)
    closes, ns = schedule(win_len, win_off, n_tok)

    def step_bytes(t):
        return L * H * sum(bm.step_bytes(D, wl.n_comp, dims.bits, wl.kda, wl.act_bf16, int(n)) for n in ns[t])

    def close_bytes_at(t):
        if gr.fused_at(t) >= 0:  # the step's token inside the close
            return L * H * sum(bm.fused_bytes(D, wl.n_comp, dims.bits, wl.kda, wl.act_bf16, int(ns[t][s]))
                               for s in closes[t])
        return L * H * sum(bm.close_bytes(D, wl.n_comp, dims.bits, wl.kda, wl.act_bf16, int(ns[t][s]) + 1)
                           for s in closes[t])

    def decode_steps(t0, t1):  # the steps in [t0, t1) taken by decode launches
        return [t for t in range(t0, t1) if gr.fused_at(t) < 0]

    # inputs resident in HBM before anything is timed
    S_init = runner.states_to_device(wk.initial_states(wl, range(wl.batch)))
    toks = [wk.device_tokens(wl, n_tok, seed=l) for l in range(L)]
    states = [lqk.State(dims) for _ in range(L)]
    outs = [torch.empty((BH, D), dtype=torch.float32, device="cuda") for _ in range(L)]
    state_tensors = [getattr(st, n) for st in states for n in lqk.STATE_FIELDS]

    def encode_all():
        for st in states:
            lqk.encode(dims, S_init, st)
        torch.cuda.synchronize()

    def check_err():
        err = int(sum(int(st.err.item()) for st in states))
        assert err == 0, f"device error word {err}"

    gr = Graphs(dims, states, toks, outs, closes, lqk, torch, ns=ns, fuse=not args.no_fuse)
    torch.cuda.synchronize()
    warm_plan, timed_plan = gr.plan(0, Wu), gr.plan(Wu, total)
    torch.cuda.synchronize()
    encode_all()  # capture ran nothing; start from freshly encoded states
    replay(warm_plan, torch, timed=False)
    torch.cuda.synchronize()
    run, walls = timed_repeats(timed_plan, state_tensors, torch, check_err)
    wall = run["wall"]

    # per-kernel averages from the events; algorithmic bytes from the schedule
    dec_us = sum(s[2] for s in run["seg"])
    close_us = sum(s[3] for s in run["seg"])
    n_dec = sum((s[1] - s[0] - int(s[5])) * L for s in run["seg"])
    n_close = sum(L for s in run["seg"] if s[4])
    n_fused = sum(L for s in run["seg"] if s[5])
    dec_bytes = sum(step_bytes(t) for t in decode_steps(Wu, total))
    close_bytes = sum(close_bytes_at(t) for t in range(Wu, total))
    # the events lie inside the wall-clock region, and no figure beats the HBM peak
    assert dec_us + close_us <= wall * 1e6 * 1.02, (dec_us, close_us, wall)
    assert (dec_bytes + close_bytes) / wall <= HBM_PEAK_GBS * 1e9, "all-in bytes above the HBM peak"
    assert dec_bytes / (dec_us * 1e-6) <= HBM_PEAK_GBS * 1e9, "decode bytes above the HBM peak"
    assert L * (dec_us / n_dec) * K <= wall * 1e6 * 1.02
    res = dict(wall=wall, walls=walls, dec_us=dec_us / n_dec, close_us=close_us / max(n_close, 1),
               n_dec=n_dec, n_close=n_close, n_fused=n_fused, dec_bytes=dec_bytes, close_bytes=close_bytes,
               dec_gbs=dec_bytes / (dec_us * 1e-6) / 1e9,
               head_tokens=K * L * BH, state_mb=states[0].nbytes() / 1e6,
               positions=positions_text([ns[t] for t in decode_steps(Wu, total)]))

    # Decode launches over whole windows: from a fresh encode, one period of the
    # close schedule runs untimed, then the next period is replayed with the same
    # per-segment graphs and events (median of three).
    pos_plan = gr.plan(0, 2 * period)
    per = []
    for _ in range(3):
        encode_all()
        replay([p for p in pos_plan if p[0] < period], torch, timed=False)
        evs = replay([p for p in pos_plan if p[0] >= period], torch, timed=True)
        torch.cuda.synchronize()
        per.append(sum(e0.elapsed_time(e1) * 1e3 for (_, _, e0, e1, _, _, _) in evs))
    us_period = float(np.median(per))
    pos_steps = decode_steps(period, 2 * period)
    pos_bytes = sum(step_bytes(t) for t in pos_steps)
    res["whole_windows"] = dict(steps=period, decode_steps=len(pos_steps),
                                avg_launch_us=us_period / (len(pos_steps) * L),
                                bytes_per_launch=pos_bytes / (len(pos_steps) * L),
                                gbs=pos_bytes / (us_period * 1e-6) / 1e9)
    check_err()
    del pos_plan

    # The same steps with the window closes overlapped: runner.capture_tokens puts
    # the close of layer l on a side stream as soon as layer l's decode is done;
    # only layer l's next decode waits for it (bit-identical results).
    lq_last = None
    if not args.no_overlap:
        del warm_plan, timed_plan, gr, states, state_tensors
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
        tens = [getattr(d.state, n) for d in decs for n in lqk.STATE_FIELDS]
        saved = [x.clone() for x in tens]
        ow = []
        for _ in range(REPEATS):
            for x, s in zip(tens, saved):
                x.copy_(s)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            g_timed.replay()
            torch.cuda.synchronize()
            ow.append(time.perf_counter() - t0)
        res["overlap_wall"] = sorted(ow)[len(ow) // 2]
        assert sum(int(d.state.err.item()) for d in decs) == 0
        lq_last = torch.stack([o.clone() for o in outs])  # outputs of the last timed step
        del decs, g_warm, g_timed, tens, saved
    else:
        lq_last = torch.stack([o.clone() for o in outs])
        del warm_plan, timed_plan, gr, states, state_tensors
    torch.cuda.synchronize()

    # FP32-state baseline on identical inputs and the same protocol
    if not args.no_fp32:
        Sf = [S_init.clone() for _ in range(L)]
        fg = Graphs(dims, Sf, toks, outs, closes, lqk, torch, kind="fp32")
        f_warm, f_timed = fg.plan(0, Wu), fg.plan(Wu, total)
        for l in range(L):
            Sf[l].copy_(S_init)
        torch.cuda.synchronize()
        replay(f_warm, torch, timed=False)
        torch.cuda.synchronize()
        frun, _ = timed_repeats(f_timed, Sf, torch)
        fus = sum(s[2] for s in frun["seg"])
        fn = sum((b - a) * L for (a, b, *_r) in frun["seg"])
        fbytes = fn * BH * bm.fp32_step_bytes(D, wl.kda, wl.act_bf16)
        assert fbytes / frun["wall"] <= HBM_PEAK_GBS * 1e9
        res.update(fp32_wall=frun["wall"], fp32_us=fus / fn, fp32_gbs=fbytes / (fus * 1e-6) / 1e9,
                   fp32_bytes_per_launch=fbytes / fn)
        # both runs saw the same inputs: the last step's outputs against the exact fp32 recurrence
        fp_last = torch.stack(outs)
        res["quality_rel_l2"] = float(torch.linalg.vector_norm(lq_last - fp_last) /
                                      torch.linalg.vector_norm(fp_last))
        del Sf, fg, f_warm, f_timed
    del toks
    torch.cuda.synchronize()
    return res


def run_single_set(args, wl, bits):
    """The same protocol with one state set (a single layer): its 78 MB fit in the
    256 MB last-level cache, so this is a cache-warm figure, reported as such."""
    import torch

    from linear_attention_recurrent_kda_amd import bytes_model as bm
    from linear_attention_recurrent_kda_amd import leapquant as lqk
    from linear_attention_recurrent_kda_amd import runner
    from linear_attention_recurrent_kda_amd import workloads as wk

    K, Wu = args.steps, args.warmup
    total = Wu + K
    dims = runner.dims_for(wl, bits)
    BH, D, H = wl.batch * wl.heads, wl.d_k, wl.heads
    win_len, win_off = wk.window_lengths(wl), wk.window_offsets(wl)
    closes, ns = schedule(win_len, win_off, total)
    st = lqk.State(dims)
    lqk.encode(dims, runner.states_to_device(wk.initial_states(wl, range(wl.batch))), st)
    toks = [wk.device_tokens(wl, total, seed=0)]
    outs = [torch.empty((BH, D), dtype=torch.float32, device="cuda")]
    gr = Graphs(dims, [st], toks, outs, closes, lqk, torch, ns=ns, fuse=not args.no_fuse)
    warm_plan, timed_plan = gr.plan(0, Wu), gr.plan(Wu, total)
    replay(warm_plan, torch, timed=False)
    torch.cuda.synchronize()
    run, _ = timed_repeats(timed_plan, [getattr(st, n) for n in lqk.STATE_FIELDS], torch)
    assert int(st.err.item()) == 0
    dec_us = sum(s[2] for s in run["seg"])
    n_dec = sum(s[1] - s[0] - int(s[5]) for s in run["seg"])
    dec_bytes = sum(H * sum(bm.step_bytes(D, wl.n_comp, dims.bits, wl.kda, wl.act_bf16, int(n)) for n in ns[t])
                    for t in range(Wu, total) if gr.fused_at(t) < 0)
    return {"note": "one state set, resident in the last-level cache: a warm figure, not the HBM measurement",
            "value": round(K * BH / run["wall"], 1), "unit": "head-tokens/s",
            "decode_avg_launch_us": round(dec_us / n_dec, 3),
            "decode_gbs": round(dec_bytes / (dec_us * 1e-6) / 1e9, 1)}


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


def run_snapshot(wl, bits, sets=8):
    """Prefix-cache snapshot and restore of every sequence at a window boundary.
    HBM-bound copies: one record per head read and written once each way. The
    timed launches rotate over `sets` state sets and snapshot buffers (as the
    decode legs rotate over layers), so that the last-level cache does not hold
    what a launch reads; one set copied again and again is reported beside it,
    labelled as cache-resident."""
    import torch

    from linear_attention_recurrent_kda_amd import leapquant as lqk
    from linear_attention_recurrent_kda_amd import runner
    from linear_attention_recurrent_kda_amd import workloads as wk

    dims = runner.dims_for(wl, bits)
    N, d = wl.batch * wl.heads, wl.d_k
    S0 = runner.states_to_device(wk.initial_states(wl, range(wl.batch)))
    sts = []
    for _ in range(sets):
        st = lqk.State(dims)
        lqk.encode(dims, S0, st)
        sts.append(st)
    del S0
    rec = lqk.snapshot_bytes(dims)
    snaps = [torch.empty((wl.batch, wl.heads, rec), dtype=torch.uint8, device="cuda") for _ in range(sets)]
    best, best_one = {}, {}
    for name, fn in (("snapshot", lqk.snapshot), ("restore", lqk.restore)):
        for one in (False, True):
            idx = [0] * sets if one else list(range(sets))
            for i in idx:  # warm-up
                fn(dims, sts[i], snaps[i])
            torch.cuda.synchronize()
            times = []
            rounds = 3  # back to back, so that host call overhead does not idle the GPU
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(rounds):
                    for i in idx:
                        fn(dims, sts[i], snaps[i])
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) * 1e3 / (rounds * sets))
            (best_one if one else best)[name] = min(times)
    for st in sts:
        assert int(st.err.item()) == 0
    moved = 2.0 * rec * N  # each record read once and written once
    gbs = moved / (best["snapshot"] * 1e-6) / 1e9
    return {"record_bytes_per_head": rec, "fp32_state_bytes_per_head": 4 * d * d,
            "heads": N, "sets": sets, "snapshot_us": round(best["snapshot"], 1), "restore_us": round(best["restore"], 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "single_set_cache_resident": {"snapshot_us": round(best_one["snapshot"], 1),
                                          "restore_us": round(best_one["restore"], 1),
                                          "note": "one state set copied again and again: held by the last-level "
                                                  "cache, not the HBM figure"}}


def cpu_baseline(wl, bits, sample):
    """The fp64 oracle (plain definition, as it stands) on a bounded sample of the
    same workload, timed twice: with the BLAS pool at its default size and
    limited to one thread. Elementwise NumPy runs on one thread either way; only
    the batched products may use more."""
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
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])

    def timed():
        t0 = time.perf_counter()
        lq.run_dense(S0, toks, np.repeat(wk.window_lengths(wl)[seqs], wl.heads),
                     np.repeat(wk.window_offsets(wl)[seqs], wl.heads), r=wl.n_comp, T=wl.power_iters,
                     bits=bits, smoothing=wl.smoothing, warm_start=wl.warm_start)
        return time.perf_counter() - t0

    dt_all = timed()
    with threadpool_limits(1):
        dt_one = timed()
    rate_all, rate_one = N * n_steps / dt_all, N * n_steps / dt_one
    full = wl.batch * wl.heads * wl.steps  # head-tokens of the whole workload
    return dict(value=round(rate_all, 1), unit="head-tokens/s", cores=threads, kind="oracle",
                sample=f"{n_seq} of {wl.batch} sequences x {wl.heads} heads x {n_steps} tokens of the same "
                       f"workload (initial encode + {n_steps // wl.window} window closes), numpy fp64, "
                       f"{dt_all:.1f} s with BLAS threads {threads}",
                single_thread={"value": round(rate_one, 1), "seconds": round(dt_one, 1), "cores": 1},
                os_cpu_count=os.cpu_count(), affinity_cores=len(os.sched_getaffinity(0)),
                full_workload_s_extrapolated=round(full / rate_all, 1))


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
    print(f"bench: {wl.name} int{bits}, {args.layers} state sets, warmup {args.warmup}, "
          f"{args.steps} timed steps x {REPEATS} repeats", file=sys.stderr, flush=True)
    r = run_gpu(args, wl, bits)
    value = r["head_tokens"] / r["wall"]
    ww = r["whole_windows"]
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
        "timing": {"repeats": REPEATS, "wall_ms_each": [round(w * 1e3, 3) for w in r["walls"]],
                   "reported": "median"},
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
            "timed_window_positions": r["positions"],
            "whole_windows": {"steps": ww["steps"], "decode_steps": ww["decode_steps"],
                              "avg_launch_us": round(ww["avg_launch_us"], 3),
                              "bytes_per_launch": round(ww["bytes_per_launch"]),
                              "achieved": round(ww["gbs"], 1), "frac": round(ww["gbs"] / HBM_PEAK_GBS, 4)},
        },
        "window_close": {"avg_launch_us": round(r["close_us"], 3), "launches": r["n_close"],
                         "bytes_per_launch": round(r["close_bytes"] / max(r["n_close"], 1)),
                         "with_last_token": r["n_fused"],
                         "note": "launches that also take the window's last token (leapquant_decode_close_at) "
                                 "are counted in with_last_token; that token has no decode launch"},
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
                                 "achieved_gbs": round(r["fp32_gbs"], 1),
                                 "frac": round(r["fp32_gbs"] / HBM_PEAK_GBS, 4),
                                 "leapquant_output_rel_l2": round(r["quality_rel_l2"], 6)}
        line["speedup_vs_fp32"] = round(value / fval, 3)
        line["speedup_decode_kernel_vs_fp32_kernel"] = round(r["fp32_us"] / r["dec_us"], 3)
    if args.prefill_tokens > 0:
        line["prefill_handoff"] = run_prefill(wl, bits, args.prefill_tokens)
    if not args.no_snapshot:
        line["snapshot"] = run_snapshot(wl, bits)
    if "fp32_us" in r:
        # the FP32 state's bytes at the HBM peak: the speedup that no FP32-state
        # kernel, however fast, could reduce the measured one below
        fp32_step_s = args.layers * r["fp32_bytes_per_launch"] / (HBM_PEAK_GBS * 1e9)
        lq_step_s = r["wall"] / args.steps
        line["speedup_vs_fp32_at_hbm_peak"] = round(fp32_step_s / lq_step_s, 3)
    if not args.no_stream_reference:
        line["stream_reference"] = stream_reference(r["dec_bytes"] // max(r["n_dec"], 1), args.layers)
    line["warm_single_set"] = run_single_set(args, wl, bits)
    line["outlier_ratio"] = outlier_report(wl, bits)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, bits, args.cpu_sample)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

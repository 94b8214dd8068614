#!/usr/bin/env python3
"""Throughput of the chunkwise mLSTMsig forward pass on one GPU.

One step = one tfla_fwd_ws call (gate prefix sums, inter-chunk states,
intra-chunk outputs) over the whole workload, inputs and workspace already
resident in HBM.  Default workload: mLSTMsig, B=4, H=8, T=8192, d_qk=256,
d_hv=512, bf16 I/O, at the best of the chunk sizes 64/128/256 (all chunk
sizes are swept and reported).  Prints one JSON line on stdout; progress
goes to stderr.

Roofline accounting (per launch, algorithmic = what the chunkwise method
must move or compute, not what the kernels happen to execute):
  flops  state kernel : 2 d_qk d_hv per step of chunks 1..N_c-1
         intra kernel : 2 d_qk d_hv per step of chunks 2..N_c  (q C_{k-1})
                        + n(n+1)(d_qk + d_hv) per chunk of n steps (causal QK^T and PV)
  bytes  gate kernel  : gate pre-activations in, a and li out (16 B per step) + g
                        (per-channel gate: also k in and the weighted keys out)
         state kernel : k, v of chunks 1..N_c-1 in, a and li in, states out (I/O type)
                        (per-channel gate: the weighted keys instead of k and a)
         intra kernel : q, k, v in, h out, states in (I/O type), a and li in
The dominant kernel (longest average duration, measured with HIP events
recorded around each launch on the stream it runs on) is reported against
the HBM peak (8 TB/s) when its arithmetic intensity is below the bf16
matrix-core ridge (2.5 PFLOP/s / 8 TB/s), else against the matrix-core peak.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mLSTMsig chunkwise fwd tokens/s at T=8192; % of bf16 MFMA peak, 1 MI355X"
PEAK_BF16 = 2.5e15      # dense bf16 matrix-core FLOP/s, MI355X
PEAK_FP32 = 157.3e12    # dense fp32 matrix-core FLOP/s
PEAK_HBM = 8.0e12       # HBM3E bytes/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- model
def chunk_lengths(T, L):
    nc = -(-T // L)
    return [min(L, T - k * L) for k in range(nc)]


def kernel_model(wl, L):
    """Algorithmic flops and bytes per launch of each kernel (whole workload)."""
    e = 2 if wl.dtype_name == "bf16" else 4
    bh = wl.B * wl.H
    n = chunk_lengths(wl.T, L)
    T, dqk, dhv = wl.T, wl.dqk, wl.dhv
    steps_state = sum(n[:-1])           # steps whose chunk feeds a materialised state
    steps_inter = sum(n[1:])            # steps that read a state
    st_bytes = e * dqk * dhv * (len(n) - 1)   # states are stored in the I/O type
    # per-step gate sums read by the consumers: a and li (mLSTMsig), a per
    # key channel (GLA), none for the closed-form fixed decay
    gstep = {0: 8, 1: 0, 2: 4 * dqk, 3: 8}[wl.variant]
    gchunk = {0: 4, 1: 0, 2: 4 * dqk, 3: 4}[wl.variant] * len(n)
    gin = {0: 8, 1: 0, 2: 4 * dqk, 3: 8}[wl.variant] * T
    gates = {"flops": 0, "bytes": bh * (gin + gstep * T + gchunk)}
    # the state walk's per-step gate reads: the per-channel gate's walk reads
    # the keys the gate kernel has weighted (k read and kw written there,
    # 2 d_qk e B per step) instead of K and the gate rows
    gwalk = gstep
    if wl.variant == 2:
        gates["bytes"] += bh * T * 2 * dqk * e
        gwalk = 0
    nst_bytes = 0
    if wl.variant == 3:
        # mLSTMexp's gate launches: a and the prefix maxima written, read back
        # with igate_pre and rewritten with the lower bound (+ 8 + 12 + 12 B per
        # step); the normaliser states are formed by the walk (4 d_qk B per
        # stored state) unless it is segmented, when k is read once more for
        # the normaliser contributions, which are written, read and turned
        # into normaliser states (3 x 4 d_qk B per chunk)
        gates["bytes"] += bh * T * 32
        if state_walk_segmented(wl, L):
            gates["bytes"] += bh * (T * dqk * e + 3 * 4 * dqk * len(n))
        else:
            nst_bytes = 4 * dqk * (len(n) - 1)
    state = {"flops": bh * 2 * dqk * dhv * steps_state,
             "bytes": bh * ((dqk + dhv) * e * steps_state + gwalk * steps_state + gchunk + st_bytes + nst_bytes)}
    intra_f = 2 * dqk * dhv * steps_inter + sum(m * (m + 1) * (dqk + dhv) for m in n)
    # mLSTMexp also reads its lower bound per step and the normaliser state per chunk
    exp_extra = (4 * T + 4 * dqk * (len(n) - 1)) if wl.variant == 3 else 0
    intra = {"flops": bh * intra_f,
             "bytes": bh * ((2 * dqk + dhv) * e * T + dhv * e * T + st_bytes + gstep * T + exp_extra)}
    return {"gates": gates, "state": state, "intra": intra}


def state_walk_segmented(wl, L):
    """Whether the library cuts the state walk into segments (few heads
    and tiles for the 256 CUs, at least four chunks feeding a state)."""
    nfeed = -(-wl.T // L) - 1
    if nfeed < 4:
        return False
    t = 128 if (wl.dtype_name == "bf16" and wl.dqk % 128 == 0 and wl.dhv % 128 == 0) else 64
    heads_tiles = wl.B * wl.H * (wl.dhv // t) * (wl.dqk // t)
    return heads_tiles < 256 and min(-(-256 // heads_tiles), nfeed // 2) >= 2


def total_flops(wl, L):
    m = kernel_model(wl, L)
    return sum(v["flops"] for v in m.values())


def backward_flops(wl, L):
    """Algorithmic flops of one backward pass (tfla_bwd): the forward states
    recomputed and the reverse state walk (2 d_qk d_hv per step of the chunks
    that feed a state, each), the three inter-chunk products of dq, dk and dv
    (2 d_qk d_hv per step that reads a state, each) and their three causal
    intra-chunk products (n(n+1)(d_qk + d_hv) per chunk of n steps, each)."""
    n = chunk_lengths(wl.T, L)
    per_head = (2 * 2 * wl.dqk * wl.dhv * sum(n[:-1]) + 3 * 2 * wl.dqk * wl.dhv * sum(n[1:])
                + 3 * sum(m * (m + 1) * (wl.dqk + wl.dhv) for m in n))
    return wl.B * wl.H * per_head


# --------------------------------------------------------------------------- GPU timing
def settle(call, seconds=0.05, batch=8):
    """Untimed calls until `seconds` have passed: the device reaches its
    steady clocks only after some tens of milliseconds of work, more than a
    few warm-up steps give."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            call()
        torch.cuda.synchronize()


def run_gpu(wl, L, steps, warmup, inputs_dev, cold_calls=0, flags=0, keep_h=False, clocks=None):
    """flags: extra variant bits (TFLA_STATES_FP32); keep_h: also return h;
    clocks: a dict that receives the clock levels read while 300 more calls
    run (after the timed pass)."""
    import torch
    from mlstm_sequence_amd import tfla

    q, k, v = inputs_dev["q"], inputs_dev["k"], inputs_dev["v"]
    ig, fg = inputs_dev["igate_pre"], inputs_dev["fgate_pre"]
    gate = {0: tfla.MLSTM_SIG, 1: tfla.SCALAR_DECAY, 2: tfla.GLA_KEY, 3: tfla.MLSTM_EXP}[wl.variant]
    var = tfla.variant_of(gate, q.dtype) | flags
    h = torch.empty((wl.B, wl.H, wl.T, wl.dhv), dtype=q.dtype, device=q.device)
    nbytes = tfla.tfla_workspace_bytes(wl.B, wl.H, wl.T, wl.dqk, wl.dhv, L, var)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()
    args = (q, k, v, ig, fg, h, wl.B, wl.H, wl.T, wl.dqk, wl.dhv, L, var, ws, nbytes)

    for _ in range(warmup):
        tfla.tfla_fwd_ws(*args)
    torch.cuda.synchronize()
    settle(lambda: tfla.tfla_fwd_ws(*args))

    # Per-kernel durations: events recorded on the launch stream between the
    # kernels (tfla_fwd_ws_marked).  The markers themselves add ~10 us per
    # step, so this pass's step time is reported separately; it also brings
    # the device to its steady state before the step time is taken.
    marks = []
    for _ in range(steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for ev in evs:
            ev.record(stream)          # creates the event; the library re-records it
        marks.append(evs)
    mstart = torch.cuda.Event(enable_timing=True)
    mend = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    mstart.record(stream)
    for i in range(steps):
        tfla.tfla_fwd_ws_marked(*args, [ev.cuda_event for ev in marks[i]])
    mend.record(stream)
    torch.cuda.synchronize()
    ms_marked = mstart.elapsed_time(mend) / steps

    # The step time: the library call itself, no instrumentation between its
    # kernels.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        tfla.tfla_fwd_ws(*args)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    if clocks is not None:
        # shader clock levels sampled every ~5 ms while 300 more calls run
        for _ in range(300):
            tfla.tfla_fwd_ws(*args)
        samples = []
        for _ in range(16):
            samples.append(sysfs_clocks())
            time.sleep(0.005)
        torch.cuda.synchronize()
        sc = sorted(int(re.sub(r"\D", "", x["sclk"])) for x in samples if x and x.get("sclk"))
        clocks["under_load"] = {"sclk_mhz_samples": sc, "mclk": (samples[0] or {}).get("mclk"),
                                "calls": 300, "ms_per_call": ms} if sc else None
    cold = None
    if cold_calls:
        # cold caches: a 1 GiB write between calls evicts the 8 x 4 MB L2 and
        # the 256 MB last-level cache; each call timed alone
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=q.device)
        times = []
        for _ in range(cold_calls):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            tfla.tfla_fwd_ws(*args)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        cold = {"median_ms": times[len(times) // 2], "min_ms": times[0], "calls": cold_calls, "flush_bytes": 1 << 30}
        del flush
    per = {"gates": 0.0, "state": 0.0, "intra": 0.0}
    for evs in marks:
        per["gates"] += evs[0].elapsed_time(evs[1])
        per["state"] += evs[1].elapsed_time(evs[2])
        per["intra"] += evs[2].elapsed_time(evs[3])
    per = {kname: t / steps for kname, t in per.items()}
    per["step_with_marks"] = ms_marked
    del ws
    return ms, wall / steps * 1e3, per, cold, (h if keep_h else None)


def run_gpu_bwd(wl, L, steps, warmup, inputs_dev, dh):
    """Milliseconds per tfla_bwd call (caller-owned workspace), timed with
    events on the stream the library launches on."""
    import torch
    from mlstm_sequence_amd import tfla

    q, k, v = inputs_dev["q"], inputs_dev["k"], inputs_dev["v"]
    ig, fg = inputs_dev["igate_pre"], inputs_dev["fgate_pre"]
    gate = {0: tfla.MLSTM_SIG, 1: tfla.SCALAR_DECAY, 2: tfla.GLA_KEY, 3: tfla.MLSTM_EXP}[wl.variant]
    var = tfla.variant_of(gate, q.dtype)
    nws = tfla.tfla_bwd_workspace_bytes(wl.B, wl.H, wl.T, wl.dqk, wl.dhv, L, var)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dig = None if ig is None else torch.empty_like(ig)
    dfg = torch.empty_like(fg)
    args = (q, k, v, ig, fg, dh, dq, dk, dv, dig, dfg, wl.B, wl.H, wl.T, wl.dqk, wl.dhv, L, var, ws, nws)
    stream = torch.cuda.current_stream()

    def timed(call):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        settle(call, batch=2)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(steps):
            call()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    ms = timed(lambda: tfla.tfla_bwd(*args))
    # training use: the forward pass ran on this workspace, and the backward
    # reuses its gate sums and states (TFLA_BWD_REUSE_FWD)
    h = torch.empty_like(v)
    tfla.tfla_fwd_ws(q, k, v, ig, fg, h, wl.B, wl.H, wl.T, wl.dqk, wl.dhv, L, var, ws, nws)
    reuse = args[:17] + (var | tfla.BWD_REUSE_FWD, ws, nws)
    ms_reuse = timed(lambda: tfla.tfla_bwd(*reuse))
    del ws, dq, dk, dv, dig, dfg, h
    return ms, ms_reuse


def run_gpu_decode(wl, steps_per_call, calls, warmup):
    """tfla_fwd_recurrent from a carried state (decoding): microseconds per
    call of `steps_per_call` steps over all B*H heads, and the HBM bytes the
    step-by-step form must move (the fp32 state read and written once per
    call, plus q, k, v, h and gates of the steps)."""
    import torch
    import workloads as W
    from mlstm_sequence_amd import tfla

    sub = wl.with_(T=steps_per_call)
    inp = W.make_inputs(sub)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    gate = {0: tfla.MLSTM_SIG, 1: tfla.SCALAR_DECAY, 2: tfla.GLA_KEY, 3: tfla.MLSTM_EXP}[wl.variant]
    var = tfla.variant_of(gate, d["q"].dtype)
    state = W.initial_state(wl.B, wl.H, wl.dqk, wl.dhv, seed=wl.seed + 2).cuda()
    h = torch.empty_like(d["v"])
    call = lambda: tfla.tfla_fwd_recurrent(d["q"], d["k"], d["v"], d["igate_pre"], d["fgate_pre"], state, h,
                                           wl.B, wl.H, steps_per_call, wl.dqk, wl.dhv, var)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    settle(call)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(calls):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / calls * 1e3
    e = 2 if wl.dtype_name == "bf16" else 4
    bh = wl.B * wl.H
    gate_bytes = {0: 8, 1: 0, 2: 4 * wl.dqk}[wl.variant] * steps_per_call * bh
    nbytes = bh * (2 * 4 * wl.dqk * wl.dhv + steps_per_call * ((2 * wl.dqk + 2 * wl.dhv) * e)) + gate_bytes
    return {"steps_per_call": steps_per_call, "us_per_call": us, "tokens_per_s": wl.B * steps_per_call / (us * 1e-6),
            "hbm_bytes_per_call": nbytes, "achieved_GBps": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / PEAK_HBM}


def roofline_for(wl, L, per):
    """The dominant kernel's (longest average duration) algorithmic bytes or
    flops per launch over its measured duration, against the HBM peak when
    its arithmetic intensity is below the bf16 matrix-core ridge, else
    against the matrix-core peak of the I/O type."""
    model = kernel_model(wl, L)
    dom = max(("gates", "state", "intra"), key=lambda k: per[k])
    dm = model[dom]
    dt = per[dom] * 1e-3
    peak_f = PEAK_BF16 if wl.dtype_name == "bf16" else PEAK_FP32
    if dm["flops"] / peak_f > dm["bytes"] / PEAK_HBM:
        roof = {"bound": "mfma", "achieved": dm["flops"] / dt / 1e12, "peak": peak_f / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": dm["bytes"] / dt / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_for(dom, wl, L)
    roof.update({"kernel": dom, "ms_per_launch": per[dom], "algorithmic_bytes": dm["bytes"],
                 "algorithmic_flops": dm["flops"]})
    return roof


def gpu_clocks():
    """Current shader and memory clocks of GPU 0 as rocm-smi reports them,
    and its power where it reports one (None where the tool is missing or
    prints nothing parseable)."""
    import subprocess
    # Under rocprofv3 (ROCPROF_* set) a child process loads the profiler's
    # tool library, which opens the device before rocm-smi's launcher
    # re-executes itself: no clock record in profiled runs.
    if any(k.startswith("ROCPROF_") for k in os.environ):
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"], capture_output=True, text=True,
                           timeout=20)
        # (a warning about low-power states can precede the JSON on stdout)
        data = json.loads(r.stdout[r.stdout.index("{"):])
    except (OSError, ValueError, subprocess.SubprocessError):
        return None
    card = next((v for k, v in data.items() if k.startswith("card")), None)
    if not isinstance(card, dict):
        return None
    pick = lambda key: next((v for k, v in card.items() if key in k.lower()), None)
    return {"sclk": pick("sclk clock speed"), "mclk": pick("mclk clock speed"), "fclk": pick("fclk clock speed"),
            "power_w": pick("power")}


def sysfs_clocks():
    """The current DPM level of the shader, memory and fabric clocks of the
    first card, read from sysfs (a file read: usable while kernels run and
    under the profiler); None where the files are missing."""
    out = {}
    for name in ("sclk", "mclk", "fclk"):
        for path in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{name}")):
            try:
                with open(path) as fh:
                    lines = fh.read().splitlines()
            except OSError:
                continue
            cur = next((ln for ln in lines if ln.strip().endswith("*")), None)
            if cur:
                out[name] = cur.split(":", 1)[1].replace("*", "").strip()
                break
    return out or None


def hbm_probe(nbytes=4 << 30, reps=10):
    """The HBM rates plain streaming kernels reach on this device over a
    buffer 16x the 256 MB last-level cache: the library's streaming probe
    (tfla_dbg_stream: 16-byte loads, a given number in flight per thread,
    a given number of 256-thread workgroups; the best of a small sweep) and
    torch's own element-wise copy and sum reduction for comparison.  The
    practical ceiling of an HBM-bound kernel, beside the 8 TB/s of the
    specification."""
    import torch
    from mlstm_sequence_amd import tfla
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    res = {"buffer_bytes": nbytes, "reps": reps}

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def entry(ms, moved, **kw):
        rate = moved / (ms * 1e-3)
        return dict(kw, ms=ms, bytes=moved, GBps=rate / 1e9, frac_of_8TBps=rate / PEAK_HBM)

    half = nbytes // 2
    sweep = []
    for loads in (4, 8, 16):
        for wgs in (256, 512, 1024, 2048):
            ms = timed(lambda: tfla.tfla_dbg_stream(0, src, dst, nbytes, loads, wgs))
            sweep.append(entry(ms, nbytes, kind="read", loads_per_thread=loads, workgroups=wgs))
    for loads in (1, 4, 8):
        for wgs in (256, 1024):
            # the first half of src copied to the first half of dst
            ms = timed(lambda: tfla.tfla_dbg_stream(1, src, dst, half, loads, wgs))
            sweep.append(entry(ms, 2 * half, kind="copy", loads_per_thread=loads, workgroups=wgs))
    res["probe_sweep"] = sweep
    res["probe_read_best"] = max((x for x in sweep if x["kind"] == "read"), key=lambda x: x["GBps"])
    res["probe_copy_best"] = max((x for x in sweep if x["kind"] == "copy"), key=lambda x: x["GBps"])
    res["torch_copy"] = entry(timed(lambda: dst.copy_(src)), 2 * nbytes)
    res["torch_read"] = entry(timed(lambda: src.sum()), nbytes)
    del src, dst
    return res


def clock_ramp(wl, L, chunks=40, per_chunk=60):
    """The step time and the shader clock level under sustained load: after
    a short warm-up and 0.5 s idle, `chunks` x `per_chunk` forward calls back
    to back, HIP events between the chunks and the sysfs clock level read
    after each chunk is enqueued."""
    import torch
    from mlstm_sequence_amd import tfla
    import workloads as W
    d = {n: (None if t is None else t.cuda()) for n, t in W.make_inputs(wl).items()}
    gate = {0: tfla.MLSTM_SIG, 1: tfla.SCALAR_DECAY, 2: tfla.GLA_KEY, 3: tfla.MLSTM_EXP}[wl.variant]
    var = tfla.variant_of(gate, d["q"].dtype)
    h = torch.empty((wl.B, wl.H, wl.T, wl.dhv), dtype=d["q"].dtype, device="cuda")
    nb = tfla.tfla_workspace_bytes(wl.B, wl.H, wl.T, wl.dqk, wl.dhv, L, var)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    args = (d["q"], d["k"], d["v"], d["igate_pre"], d["fgate_pre"], h, wl.B, wl.H, wl.T, wl.dqk, wl.dhv, L, var,
            ws, nb)
    for _ in range(5):
        tfla.tfla_fwd_ws(*args)
    torch.cuda.synchronize()
    time.sleep(0.5)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(chunks + 1)]
    evs[0].record()
    t0 = time.perf_counter()
    samples = []
    for c in range(chunks):
        for _ in range(per_chunk):
            tfla.tfla_fwd_ws(*args)
        evs[c + 1].record()
        samples.append(((time.perf_counter() - t0) * 1e3, sysfs_clocks()))
    torch.cuda.synchronize()
    return [{"chunk": c, "ms_per_call": evs[c].elapsed_time(evs[c + 1]) / per_chunk,
             "host_ms_at_enqueue": round(samples[c][0], 1), "clocks": samples[c][1]} for c in range(chunks)]


def mfma_probe(iters=2000, reps=5):
    """The rate the matrix cores reach on back-to-back 32x32x16 bf16
    instructions with register operands (tfla_dbg_mfma: four accumulator
    chains per wavefront, 256-thread workgroups; the best of a few grid
    sizes), beside the specification's 2.5 PFLOP/s dense bf16."""
    import torch
    from mlstm_sequence_amd import tfla
    sink = torch.zeros(1024, dtype=torch.float32, device="cuda")
    sweep = []
    for wgs in (256, 512, 1024, 2048):
        for _ in range(2):
            tfla.tfla_dbg_mfma(iters, wgs, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            tfla.tfla_dbg_mfma(iters, wgs, sink)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        flops = wgs * 4 * 4 * iters * 32768
        sweep.append({"workgroups": wgs, "iters": iters, "ms": ms, "flops": flops,
                      "TFLOPs": flops / (ms * 1e-3) / 1e12, "frac_of_2.5PF": flops / (ms * 1e-3) / PEAK_BF16})
    best = max(sweep, key=lambda x: x["TFLOPs"])
    return {"sweep": sweep, "best": best}


LDS_PROBE_MODES = {0: "16-byte row reads", 1: "transpose reads", 2: "16-byte row reads, each feeding one 32x32x16",
                   3: "transpose reads, each feeding one 32x32x16", 4: "32x32x16 on a register operand"}


def lds_probe(iters=4000, reps=3):
    """How fast a CU serves the intra-chunk kernels' LDS operand reads, alone
    and each feeding one 32x32x16 bf16 instruction (tfla_dbg_lds: one
    workgroup per CU, 256 workgroups; cycles from the shader clock inside
    each workgroup, median over workgroups, best of `reps` launches).  At
    2.5 PFLOP/s a CU completes one such instruction per SIMD every 32 cycles,
    and an instruction whose A operand comes from LDS takes 1 KB of it: 128
    bytes per cycle per CU at full rate."""
    import torch
    from mlstm_sequence_amd import tfla
    n = 256
    clocks = torch.zeros(2 * n, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1024, dtype=torch.float32, device="cuda")
    out = []
    for waves in (4, 8):
        for mode in range(5):
            best = None
            for _ in range(reps + 1):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                tfla.tfla_dbg_lds(mode, waves, iters, n, clocks, sink)
                e1.record()
                torch.cuda.synchronize()
                c = clocks.view(n, 2).cpu()
                cyc = sorted((c[:, 1] - c[:, 0]).tolist())
                r = (cyc[n // 2], cyc[0], cyc[-1], e0.elapsed_time(e1))
                if best is None or r[0] < best[0]:
                    best = r
            med, lo, hi, ms = best
            lds_bytes = waves * iters * 8 * 1024 if mode < 4 else 0
            mfma = waves * iters * 8 if mode >= 2 else 0
            out.append({"mode": mode, "what": LDS_PROBE_MODES[mode], "waves": waves, "iters": iters,
                        "cycles_median": med, "cycles_min": lo, "cycles_max": hi, "launch_ms": ms,
                        "lds_bytes_per_cycle_per_cu": lds_bytes / med,
                        "mfma_busy": mfma * 32 / (med * 4)})
    return out


def measured_peaks():
    """Short probes for the bench line: the matrix cores' bf16 rate and the
    HBM read rate of the streaming probe (8 loads per thread, one
    workgroup per CU, 2 GiB)."""
    import torch
    from mlstm_sequence_amd import tfla
    m = mfma_probe(iters=1000, reps=3)["best"]
    n = 2 << 30
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    sink = torch.empty(1024, dtype=torch.float32, device="cuda")
    for _ in range(3):
        tfla.tfla_dbg_stream(0, src, sink, n, 8, 256)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        tfla.tfla_dbg_stream(0, src, sink, n, 8, 256)
    e1.record()
    torch.cuda.synchronize()
    gbps = n / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e9
    del src
    return {"mfma_bf16_tflops": m["TFLOPs"], "mfma_workgroups": m["workgroups"], "hbm_read_gbps": gbps}


# --------------------------------------------------------------------------- CPU baseline
def cpu_baseline(wl, target_s=15.0):
    """The oracle (plain C recurrence in double, OpenMP over heads) on all
    heads of the workload for its first T' steps; its cost is linear in T', so
    tokens/s over T' is its throughput on the whole sequence."""
    import oracle
    import workloads as W

    def run(Tp):
        sub = wl.with_(T=Tp)
        inp = W.make_inputs(sub)
        arrs = [W.as_f64(inp[n]) for n in ("q", "k", "v", "igate_pre", "fgate_pre")]
        t0 = time.perf_counter()
        oracle.recurrent_fwd(*arrs, wl.variant)
        return time.perf_counter() - t0

    t_cal = run(256)
    Tp = int(min(wl.T, max(256, 256 * round(target_s / max(t_cal, 1e-3)))))
    Tp = min(wl.T, (Tp // 256) * 256 or 256)
    dt = run(Tp) if Tp != 256 else t_cal
    threads = oracle.threads()
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": wl.B * Tp / dt, "unit": "tokens/s", "cores": min(threads, wl.B * wl.H),
            "kind": "oracle", "seconds": round(dt, 3), "host_threads": threads, "cpu_model": model,
            "sample": f"all {wl.B * wl.H} (b,h) heads of the workload, first {Tp} of {wl.T} steps "
                      f"(seed-identical inputs); OpenMP over heads, {min(threads, wl.B * wl.H)} threads busy"}


def traffic_for(kernel, wl, L):
    """HBM bytes per launch from committed rocprofv3 counter summaries, only
    when they were taken on the current source of that kernel."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    key = f"{kernel}:{wl.name}:L{L}"
    r = rec.get(key)
    if not r or r.get("src_sha") != source_sha(kernel):
        return None
    return r.get("bytes_per_launch")


def source_sha(kernel):
    files = {"gates": ["gates.hip"], "state": ["state.hip"], "intra": ["intra.hip", "intra_impl.hpp", "intra_sweep.hip"]}[kernel]
    hs = hashlib.sha256()
    for f in files + ["gfx950.hpp"]:
        with open(os.path.join(ROOT, "mlstm_sequence_amd", "csrc", f), "rb") as fh:
            hs.update(fh.read())
    return hs.hexdigest()[:16]


# --------------------------------------------------------------------------- HBM byte counters
def counter_run(wl, L, calls):
    """Only `calls` forward calls at chunk size L, nothing else of this
    library on the device (the target of the rocprofv3 --pmc passes that
    count HBM bytes per phase)."""
    import torch
    from mlstm_sequence_amd import tfla
    import workloads as W

    dev = {n: (None if t is None else t.cuda()) for n, t in W.make_inputs(wl).items()}
    gate = {0: tfla.MLSTM_SIG, 1: tfla.SCALAR_DECAY, 2: tfla.GLA_KEY, 3: tfla.MLSTM_EXP}[wl.variant]
    var = tfla.variant_of(gate, dev["q"].dtype)
    h = torch.empty((wl.B, wl.H, wl.T, wl.dhv), dtype=dev["q"].dtype, device="cuda")
    nbytes = tfla.tfla_workspace_bytes(wl.B, wl.H, wl.T, wl.dqk, wl.dhv, L, var)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    for i in range(calls):
        tfla.tfla_fwd_ws(dev["q"], dev["k"], dev["v"], dev["igate_pre"], dev["fgate_pre"], h,
                         wl.B, wl.H, wl.T, wl.dqk, wl.dhv, L, var, ws, nbytes)
        torch.cuda.synchronize()
        log(f"counter run: call {i + 1} of {calls} done")
    print(json.dumps({"workload": wl.name, "L": L, "calls": calls}), flush=True)


COPY_CAL_BYTES = 1 << 30


def copy_calibration():
    """A plain copy of COPY_CAL_BYTES with the streaming probe's copy kernel,
    three times: what FETCH_SIZE and WRITE_SIZE read for bytes known to
    move (the scale of the counters)."""
    import torch
    from mlstm_sequence_amd import tfla
    src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        tfla.tfla_dbg_stream(1, src, dst, COPY_CAL_BYTES, 4, 1024)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_CAL_BYTES, "dispatches": 3}), flush=True)


def _phase_of(kernel_name):
    """Phase of one of this library's forward kernels from its demangled
    name: gates, state, intra, the calibration copy, or None."""
    import re
    m = re.search(r"tfla::(?:\(anonymous namespace\)::)?(\w+)", kernel_name)
    if m:
        base = m.group(1)
    else:
        # template instances keep their mangled name: length-prefixed identifier
        m = re.search(r"_ZN4tfla12_GLOBAL__N_1(\d+)", kernel_name)
        if not m:
            return None
        base = kernel_name[m.end():m.end() + int(m.group(1))]
    if base.startswith("gates_"):
        return "gates"
    if base in ("state_kernel", "state_combine_kernel", "state_fixup_kernel"):
        return "state"
    if base.startswith("intra_kernel"):
        return "intra"
    if base == "probe_copy_kernel":
        return "copy"
    return None


def _counter_sums(csv_path, counter):
    """Sum of one counter per phase over the run, and dispatches per phase."""
    import csv
    sums, counts = {}, {}
    with open(csv_path, newline="") as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            ph = _phase_of(row["Kernel_Name"])
            if ph is None:
                continue
            sums[ph] = sums.get(ph, 0.0) + float(row["Counter_Value"])
            counts[ph] = counts.get(ph, 0) + 1
    return sums, counts


def write_traffic(run_dir, wl, L, out_path=None):
    """HBM bytes per forward launch of each phase from four rocprofv3 --pmc
    runs under run_dir: fetch/ and write/ (FETCH_SIZE, WRITE_SIZE of
    --counter-run), copy_fetch/ and copy_write/ (the same counters of
    --copy-calibration).  Each counter is scaled by bytes moved over what
    it reads for the calibration copy; the per-launch figures go into
    profiles/traffic.json with the hash of each kernel's source, and a
    markdown table is printed."""
    csvp = lambda sub: os.path.join(run_dir, sub, "run_counter_collection.csv")
    cf, nf = _counter_sums(csvp("copy_fetch"), "FETCH_SIZE")
    cw, nw = _counter_sums(csvp("copy_write"), "WRITE_SIZE")
    # a copy moves the bytes once in each direction; counters in KiB
    fetch_scale = COPY_CAL_BYTES / (cf["copy"] / nf["copy"] * 1024)
    write_scale = COPY_CAL_BYTES / (cw["copy"] / nw["copy"] * 1024)
    fs, fn = _counter_sums(csvp("fetch"), "FETCH_SIZE")
    ws_, wn = _counter_sums(csvp("write"), "WRITE_SIZE")
    calls = fn["intra"]
    if wn.get("intra") != calls:
        raise SystemExit(f"fetch and write runs differ in forward calls ({calls} vs {wn.get('intra')})")
    model = kernel_model(wl, L)
    path = out_path or os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    print(f"Calibration: a {COPY_CAL_BYTES >> 20} MiB copy reads FETCH_SIZE = {cf['copy'] / nf['copy']:.0f} KiB "
          f"and WRITE_SIZE = {cw['copy'] / nw['copy']:.0f} KiB per dispatch: fetch scale {fetch_scale:.3f}, "
          f"write scale {write_scale:.3f}; {calls} forward calls.\n")
    print("| phase | dispatches per call | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB "
          "| total MB | algorithmic MB | total / algorithmic |")
    print("|---|---|---|---|---|---|---|---|---|")
    for ph in ("gates", "state", "intra"):
        if ph not in fs:
            continue
        fk, wk = fs[ph] / calls, ws_.get(ph, 0.0) / calls
        fb, wb = fk * 1024 * fetch_scale, wk * 1024 * write_scale
        alg = model[ph]["bytes"]
        rec[f"{ph}:{wl.name}:L{L}"] = {
            "bytes_per_launch": fb + wb, "fetch_bytes": fb, "write_bytes": wb, "fetch_kib_counter": fk,
            "write_kib_counter": wk, "fetch_scale": fetch_scale, "write_scale": write_scale,
            "algorithmic_bytes": alg, "calls": calls, "src_sha": source_sha(ph)}
        print(f"| {ph} | {fn[ph] // calls} | {fk:.0f} | {wk:.0f} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | "
              f"{(fb + wb) / 1e6:.1f} | {alg / 1e6:.1f} | {(fb + wb) / alg:.3f} |")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
        fh.write("\n")


# --------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload index (1..5)")
    ap.add_argument("--L", type=int, default=None, help="headline chunk size (default: best listed)")
    ap.add_argument("--sweep", type=str, default=None, help="comma-separated chunk sizes to sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--no-fp32-states", action="store_true",
                    help="skip the timing with the states materialised in fp32 (TFLA_STATES_FP32)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (scales HBM byte counters)")
    ap.add_argument("--counter-run", action="store_true",
                    help="only warmup + steps forward calls at --L (target of the HBM byte counter runs)")
    ap.add_argument("--traffic-from", type=str, default=None, metavar="DIR",
                    help="no GPU: turn the FETCH_SIZE/WRITE_SIZE runs under DIR into per-launch HBM bytes "
                         "of --config at --L (profiles/traffic.json) and print them")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="only measure the HBM rate of plain streaming kernels (copy, read) and print it")
    ap.add_argument("--probe-mib", type=str, default="4096",
                    help="--hbm-probe buffer sizes in MiB, comma-separated (sizes within the 256 MB "
                         "last-level cache show what it serves)")
    ap.add_argument("--probe-reps", type=int, default=10, help="--hbm-probe timed calls per point")
    ap.add_argument("--clock-ramp", action="store_true",
                    help="step time and shader clock level through ~1 s of back-to-back calls of --config at "
                         "--L (default 256), then exit")
    ap.add_argument("--lds-probe", action="store_true",
                    help="LDS operand-read rates alone and feeding the matrix cores (tfla_dbg_lds), then exit")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only measure the bf16 matrix-core rate of back-to-back instructions and print it")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads' lines (default workload only)")
    args = ap.parse_args()

    if args.copy_calibration:
        copy_calibration()
        return
    if args.traffic_from or args.counter_run:
        import workloads as W
        wl = W.WORKLOADS[args.config]
        if args.L is None:
            raise SystemExit("--counter-run and --traffic-from need --L")
        if args.traffic_from:
            write_traffic(args.traffic_from, wl, args.L)
        else:
            counter_run(wl, args.L, args.warmup + args.steps)
        return

    if args.clock_ramp:
        import workloads as W
        for x in clock_ramp(W.WORKLOADS[args.config], args.L or 256):
            log(f"chunk {x['chunk']:2d}: {x['ms_per_call']:.4f} ms/call, enqueued by {x['host_ms_at_enqueue']} ms, "
                f"clocks {x['clocks']}")
            print(json.dumps(x), flush=True)
        return
    if args.hbm_probe:
        for mib in (int(x) for x in args.probe_mib.split(",")):
            r = hbm_probe(nbytes=mib << 20, reps=args.probe_reps)
            rb, cb = r["probe_read_best"], r["probe_copy_best"]
            log(f"{mib} MiB: read {rb['GBps']:.0f} GB/s ({rb['loads_per_thread']} loads per thread, "
                f"{rb['workgroups']} workgroups), copy {cb['GBps']:.0f} GB/s")
            print(json.dumps({"hbm_probe": r}), flush=True)
        return
    if args.lds_probe:
        for r in lds_probe():
            print(json.dumps({"lds_probe": r}), flush=True)
        return
    if args.mfma_probe:
        print(json.dumps({"mfma_probe": mfma_probe()}), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); every head "
              "is independent, so the per-GPU shard of a multi-GPU run is this same kernel at fewer heads",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W

    wl = W.WORKLOADS[args.config]

    listed = list(wl.chunk_sizes)
    sweep = [int(x) for x in args.sweep.split(",")] if args.sweep else sorted(
        set(listed + ([512, 1024] if args.config == 3 else [])))
    if args.L is not None and args.L not in sweep:
        sweep.append(args.L)

    log(f"workload {wl.name}: B={wl.B} H={wl.H} T={wl.T} d_qk={wl.dqk} d_hv={wl.dhv} {wl.dtype_name}; "
        f"chunk sizes {sweep}")
    inputs = W.make_inputs(wl)
    dev = {n: (None if t is None else t.cuda()) for n, t in inputs.items()}
    torch.cuda.synchronize()

    clocks_before = gpu_clocks()
    results = {}
    clocks_load = {}
    for L in sweep:
        ms, wall_ms, per, cold, _ = run_gpu(wl, L, args.steps, args.warmup, dev, cold_calls=10,
                                            clocks=clocks_load.setdefault(L, {}))
        tps = wl.B * wl.T / (ms * 1e-3)
        fl = total_flops(wl, L)
        results[L] = {"ms": ms, "wall_ms": wall_ms, "per": per, "tokens_per_s": tps,
                      "mfma_frac": fl / (ms * 1e-3) / PEAK_BF16, "cold": cold}
        log(f"L={L}: {ms:.3f} ms/step, {tps:.4g} tokens/s, {results[L]['mfma_frac'] * 100:.2f}% of bf16 peak "
            f"(gates {per['gates']:.3f} ms, state {per['state']:.3f} ms, intra {per['intra']:.3f} ms)")

    if args.L is not None:
        Lh = args.L
    else:
        Lh = max((L for L in listed if L in results), key=lambda L: results[L]["tokens_per_s"])
    r = results[Lh]
    roof = roofline_for(wl, Lh, r["per"])
    clocks_after = gpu_clocks()

    out = {
        "metric": METRIC,
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype_name,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "d_qk": wl.dqk, "d_hv": wl.dhv,
                   "L": Lh, "variant": W.VARIANT_NAMES[wl.variant], "io": wl.dtype_name},
        "mfma_frac": r["mfma_frac"],
        "roofline": roof,
        "kernels_ms": r["per"],
        "sweep": {str(L): {"tokens_per_s": x["tokens_per_s"], "ms_per_step": x["ms"],
                           "mfma_frac": x["mfma_frac"], "kernels_ms": x["per"], "cold_cache": x["cold"]}
                  for L, x in results.items()},
        "cold_cache": r["cold"],
        "gpu_clocks": {"before_sweep": clocks_before, "after_sweep": clocks_after,
                       "under_load": clocks_load.get(Lh, {}).get("under_load")},
    }
    # the matrix-core and HBM rates plain probe kernels reach on this device,
    # and the headline against them (beside the specification's peaks)
    mp = measured_peaks()
    mp["step_mfma_frac_of_measured"] = r["mfma_frac"] * PEAK_BF16 / (mp["mfma_bf16_tflops"] * 1e12)
    if roof["unit"] == "GB/s":
        mp["roofline_achieved_frac_of_measured_read"] = roof["achieved"] / mp["hbm_read_gbps"]
    out["measured_peaks"] = mp
    log(f"measured peaks: {mp['mfma_bf16_tflops']:.0f} TFLOP/s bf16 matrix cores, {mp['hbm_read_gbps']:.0f} GB/s "
        f"HBM read; step at {100 * mp['step_mfma_frac_of_measured']:.1f}% of the measured matrix-core rate")
    # mLSTMexp on the same inputs and launch (TFLA research-map summary, Key
    # results: the mLSTMsig forward kernel is over 30% faster than
    # mLSTMexp's on H100): the same state walk and intra-chunk products plus
    # its max-state chain, normaliser and bound
    if wl.variant == W.MLSTM_SIG and wl.dtype_name == "bf16":
        wle = wl.with_(variant=W.MLSTM_EXP, name=wl.name.replace("mlstm_sig", "mlstm_exp"))
        mse, _, pere, _, _ = run_gpu(wle, Lh, args.steps, args.warmup, dev)
        out["mlstm_exp"] = {"L": Lh, "ms_per_step": mse, "tokens_per_s": wl.B * wl.T / (mse * 1e-3),
                            "kernels_ms": pere, "mlstm_sig_ms_per_step": r["ms"],
                            "sig_faster_by": mse / r["ms"] - 1.0}
        log(f"mLSTMexp, L={Lh}: {mse:.3f} ms/step (gates {pere['gates']:.3f}, state {pere['state']:.3f}, "
            f"intra {pere['intra']:.3f} ms); mLSTMsig faster by {100 * (mse / r['ms'] - 1):.1f}%")
    # every other workload at its listed chunk sizes (parity cases of the
    # tests; reported so each config has a driver-run record)
    if args.config == 3 and not args.no_workloads:
        others = {}
        for c in (1, 2, 4, 5):
            wlc = W.WORKLOADS[c]
            devc = {n: (None if t is None else t.cuda()) for n, t in W.make_inputs(wlc).items()}
            for L in wlc.chunk_sizes:
                msc, _, perc, _, _ = run_gpu(wlc, L, args.steps, args.warmup, devc)
                others[f"{wlc.name}:L{L}"] = {
                    "config": c, "L": L, "B": wlc.B, "H": wlc.H, "T": wlc.T, "d_qk": wlc.dqk, "d_hv": wlc.dhv,
                    "io": wlc.dtype_name, "ms_per_step": msc, "tokens_per_s": wlc.B * wlc.T / (msc * 1e-3),
                    "mfma_frac": total_flops(wlc, L) / (msc * 1e-3) / PEAK_BF16, "kernels_ms": perc,
                    "roofline": roofline_for(wlc, L, perc)}
                log(f"{wlc.name} L={L}: {msc:.3f} ms/step, {wlc.B * wlc.T / (msc * 1e-3):.4g} tokens/s "
                    f"(gates {perc['gates']:.3f}, state {perc['state']:.3f}, intra {perc['intra']:.3f} ms)")
            del devc
        out["workloads"] = others
    # The same step with the chunk states materialised in fp32 instead of the
    # I/O type (TFLA_STATES_FP32): identical h, twice the state bytes.
    if wl.dtype_name == "bf16" and not args.no_fp32_states:
        from mlstm_sequence_amd import tfla
        _, _, _, _, h16 = run_gpu(wl, Lh, 2, 1, dev, keep_h=True)
        ms32, _, per32, _, h32 = run_gpu(wl, Lh, args.steps, args.warmup, dev, flags=tfla.STATES_FP32, keep_h=True)
        out["fp32_states"] = {"L": Lh, "ms_per_step": ms32, "tokens_per_s": wl.B * wl.T / (ms32 * 1e-3),
                              "mfma_frac": total_flops(wl, Lh) / (ms32 * 1e-3) / PEAK_BF16, "kernels_ms": per32,
                              "h_bitwise_equal": bool(torch.equal(h16, h32))}
        del h16, h32
        log(f"fp32 states, L={Lh}: {ms32:.3f} ms/step (state {per32['state']:.3f} ms, intra {per32['intra']:.3f} ms); "
            f"h bitwise equal to the bf16-state step: {out['fp32_states']['h_bitwise_equal']}")
    # Chunk-size ablation (limit_chunk vs xl_chunk, TFLA abstract and summary):
    # at L = 64 every chunk is a single 64-step key/value tile, i.e. the chunk
    # is bounded by what one workgroup stages on chip; larger L tile the
    # chunk along the sequence.  Reported when L = 64 was swept.
    if 64 in results and len(results) > 1:
        xl = max((L for L in results if L != 64), key=lambda L: results[L]["tokens_per_s"])
        out["chunking_ablation"] = {
            "limit_chunk": {"L": 64, "ms_per_step": results[64]["ms"], "tokens_per_s": results[64]["tokens_per_s"]},
            "xl_chunk": {"L": xl, "ms_per_step": results[xl]["ms"], "tokens_per_s": results[xl]["tokens_per_s"]},
            "xl_speedup": results[xl]["tokens_per_s"] / results[64]["tokens_per_s"],
        }
    # The backward pass (tfla_bwd) on the same workload, every swept chunk
    # size: context beside the forward metric, not part of `value`.
    if not args.no_backward:
        dh = W.upstream_grad(wl.B, wl.H, wl.T, wl.dhv, wl.dtype, seed=wl.seed + 1).cuda()
        bwd = {}
        for L in sweep:
            ms, ms_reuse = run_gpu_bwd(wl, L, max(1, args.steps // 2), max(1, args.warmup // 2), dev, dh)
            fl = backward_flops(wl, L)
            bwd[L] = {"ms_per_step": ms, "tokens_per_s": wl.B * wl.T / (ms * 1e-3),
                      "mfma_frac": fl / (ms * 1e-3) / PEAK_BF16, "algorithmic_flops": fl,
                      "ms_per_step_reusing_forward_states": ms_reuse}
            log(f"backward L={L}: {ms:.3f} ms/step, {bwd[L]['tokens_per_s']:.4g} tokens/s, "
                f"{bwd[L]['mfma_frac'] * 100:.2f}% of bf16 peak; {ms_reuse:.3f} ms reusing the forward's states")
        Lb = min(bwd, key=lambda L: bwd[L]["ms_per_step"])
        out["backward"] = dict(bwd[Lb], L=Lb, sweep={str(L): x for L, x in bwd.items()})
        del dh
    # Decoding with the step-by-step form (context beside the metric): one
    # step and 16 steps per call from a carried fp32 state, every head.
    out["decode"] = [run_gpu_decode(wl, n, 50, 5) for n in (1, 16)]
    for x in out["decode"]:
        log(f"decode {x['steps_per_call']} step(s)/call: {x['us_per_call']:.1f} us, "
            f"{x['achieved_GBps']:.0f} GB/s ({100 * x['hbm_frac']:.1f}% of HBM peak)")
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(wl)
        log(f"oracle: {out['cpu_baseline']['value']:.4g} tokens/s ({out['cpu_baseline']['sample']})")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

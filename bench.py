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
         state kernel : k, v of chunks 1..N_c-1 in, a and li in, states out (I/O type)
         intra kernel : q, k, v in, h out, states in (I/O type), a and li in
The dominant kernel (longest average duration, measured with HIP events
recorded around each launch on the stream it runs on) is reported against
the HBM peak (8 TB/s) when its arithmetic intensity is below the bf16
matrix-core ridge (2.5 PFLOP/s / 8 TB/s), else against the matrix-core peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
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
    gstep = {0: 8, 1: 0, 2: 4 * dqk}[wl.variant]
    gchunk = {0: 4, 1: 0, 2: 4 * dqk}[wl.variant] * len(n)
    gin = {0: 8, 1: 0, 2: 4 * dqk}[wl.variant] * T
    gates = {"flops": 0, "bytes": bh * (gin + gstep * T + gchunk)}
    state = {"flops": bh * 2 * dqk * dhv * steps_state,
             "bytes": bh * ((dqk + dhv) * e * steps_state + gstep * steps_state + gchunk + st_bytes)}
    intra_f = 2 * dqk * dhv * steps_inter + sum(m * (m + 1) * (dqk + dhv) for m in n)
    intra = {"flops": bh * intra_f,
             "bytes": bh * ((2 * dqk + dhv) * e * T + dhv * e * T + st_bytes + gstep * T)}
    return {"gates": gates, "state": state, "intra": intra}


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


def run_gpu(wl, L, steps, warmup, inputs_dev, cold_calls=0, flags=0, keep_h=False):
    """flags: extra variant bits (TFLA_STATES_FP32); keep_h: also return h."""
    import torch
    from mlstm_sequence_amd import tfla

    q, k, v = inputs_dev["q"], inputs_dev["k"], inputs_dev["v"]
    ig, fg = inputs_dev["igate_pre"], inputs_dev["fgate_pre"]
    gate = {0: tfla.MLSTM_SIG, 1: tfla.SCALAR_DECAY, 2: tfla.GLA_KEY}[wl.variant]
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
    gate = {0: tfla.MLSTM_SIG, 1: tfla.SCALAR_DECAY, 2: tfla.GLA_KEY}[wl.variant]
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
    gate = {0: tfla.MLSTM_SIG, 1: tfla.SCALAR_DECAY, 2: tfla.GLA_KEY}[wl.variant]
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
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "dispatches": 3}), flush=True)
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

    results = {}
    for L in sweep:
        ms, wall_ms, per, cold, _ = run_gpu(wl, L, args.steps, args.warmup, dev, cold_calls=10)
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
    model = kernel_model(wl, Lh)
    dom = max(("gates", "state", "intra"), key=lambda k: r["per"][k])
    dm = model[dom]
    dt = r["per"][dom] * 1e-3
    peak_f = PEAK_BF16 if wl.dtype_name == "bf16" else PEAK_FP32
    mfma_bound = dm["flops"] / peak_f > dm["bytes"] / PEAK_HBM
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": dm["flops"] / dt / 1e12, "peak": peak_f / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": dm["bytes"] / dt / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    tr = traffic_for(dom, wl, Lh)
    roof["traffic"] = tr
    roof.update({"kernel": dom, "ms_per_launch": r["per"][dom], "algorithmic_bytes": dm["bytes"],
                 "algorithmic_flops": dm["flops"]})

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
    }
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

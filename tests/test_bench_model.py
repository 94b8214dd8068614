"""The benchmark's algorithmic work model against the closed form it
implements (host logic, no GPU)."""
import pytest

import bench
import workloads as W


def f_alg(B, H, T, L, dqk, dhv):
    """Chunkwise algorithmic flops when L divides T: the state update and the
    inter term (2 d_qk d_hv each per step of the T - L steps that feed or read
    a materialised state) and the causal QK^T and PV (L(L+1)/2 pairs per
    chunk, 2 (d_qk + d_hv) flops per pair)."""
    return B * H * (4 * (T - L) * dqk * dhv + T * (L + 1) * (dqk + dhv))


@pytest.mark.parametrize("c", sorted(W.WORKLOADS))
def test_forward_flops_match_closed_form(c):
    wl = W.WORKLOADS[c]
    for L in wl.chunk_sizes:
        assert bench.total_flops(wl, L) == f_alg(wl.B, wl.H, wl.T, L, wl.dqk, wl.dhv)


def test_forward_flops_ragged_tail():
    wl = W.WORKLOADS[3].with_(T=1000)
    n = [256, 256, 256, 232]
    want = wl.B * wl.H * (2 * wl.dqk * wl.dhv * (sum(n[:-1]) + sum(n[1:]))
                          + sum(m * (m + 1) * (wl.dqk + wl.dhv) for m in n))
    assert bench.total_flops(wl, 256) == want


def test_backward_flops():
    wl = W.WORKLOADS[3]
    L = 256
    # two state walks + three inter products (2 d_qk d_hv per step each) and three causal products
    want = wl.B * wl.H * (5 * 2 * (wl.T - L) * wl.dqk * wl.dhv + 3 * wl.T * (L + 1) * (wl.dqk + wl.dhv))
    assert bench.backward_flops(wl, L) == want


def test_intra_bytes_are_compulsory_io_plus_states():
    wl = W.WORKLOADS[3]
    L = 256
    m = bench.kernel_model(wl, L)
    bh = wl.B * wl.H
    nc = wl.T // L
    io = bh * wl.T * (2 * wl.dqk + 2 * wl.dhv) * 2          # q, k, v in, h out (bf16)
    states = bh * (nc - 1) * wl.dqk * wl.dhv * 2            # states (stored bf16) read once
    gates = bh * wl.T * 8                                   # a and li
    assert m["intra"]["bytes"] == io + states + gates


# ---------------------------------------------------------------- counter summaries
def _write_counters(path, rows):
    import csv
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, counter, value) in enumerate(rows):
            w.writerow([i, name, counter, value])


def test_traffic_summary_from_counter_runs(tmp_path):
    """bench.py --traffic-from: the phase of each dispatch from its kernel
    name (demangled or mangled template instance), counters summed per phase
    and divided by the calls, scaled by the calibration copy's reading."""
    copy = "void tfla::(anonymous namespace)::probe_copy_kernel<4>(unsigned int __vector(4) const*)"
    gates = "tfla::(anonymous namespace)::gates_sig_kernel(float const*, float const*)"
    state = "_ZN4tfla12_GLOBAL__N_112state_kernelIDF16bLi0ELi128ELi128ELi128ELi8ELb0EDF16bEEvPKT_"
    fixup = "_ZN4tfla12_GLOBAL__N_118state_fixup_kernelILi0EDF16bEEvPT0_PKfS5_PfS5_S5_iiiiiiiiii"
    intra = "_ZN4tfla12_GLOBAL__N_118intra_kernel_sweepIDF16bLi0ELi256ELi8EDF16bLb0EEEvPKT_"
    other = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>"
    cal = bench.COPY_CAL_BYTES // 1024
    # a copy that the counters read at half its bytes (fetch) and in full (write)
    _write_counters(tmp_path / "copy_fetch" / "run_counter_collection.csv", [(copy, "FETCH_SIZE", cal / 2)] * 3)
    _write_counters(tmp_path / "copy_write" / "run_counter_collection.csv", [(copy, "WRITE_SIZE", cal)] * 3)
    fetch, write = [], []
    for _ in range(2):   # two forward calls
        fetch += [(gates, "FETCH_SIZE", 10), (state, "FETCH_SIZE", 100), (fixup, "FETCH_SIZE", 20),
                  (intra, "FETCH_SIZE", 300), (other, "FETCH_SIZE", 5000)]
        write += [(gates, "WRITE_SIZE", 1), (state, "WRITE_SIZE", 40), (fixup, "WRITE_SIZE", 4),
                  (intra, "WRITE_SIZE", 50), (other, "WRITE_SIZE", 5000)]
    _write_counters(tmp_path / "fetch" / "run_counter_collection.csv", fetch)
    _write_counters(tmp_path / "write" / "run_counter_collection.csv", write)
    out = tmp_path / "traffic.json"
    wl = W.WORKLOADS[3]
    bench.write_traffic(str(tmp_path), wl, 256, out_path=str(out))
    import json
    rec = json.load(open(out))
    st = rec[f"state:{wl.name}:L256"]
    assert st["fetch_bytes"] == pytest.approx(2 * 120 * 1024)   # fetch scale 2
    assert st["write_bytes"] == pytest.approx(44 * 1024)
    assert rec[f"intra:{wl.name}:L256"]["bytes_per_launch"] == pytest.approx((2 * 300 + 50) * 1024)
    assert rec[f"gates:{wl.name}:L256"]["calls"] == 2
    assert st["src_sha"] == bench.source_sha("state")

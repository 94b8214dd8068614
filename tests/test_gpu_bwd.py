"""The backward pass (tfla_bwd) through the C ABI against the oracle's
backward recurrence, element by element, on seeded inputs.

Gradients of L = sum(dh * h) with respect to q, k, v and the gate
pre-activations; tolerance max|d|/max|ref| <= 1e-4 (fp32 I/O) and <= 2e-2
(bf16 I/O) on every gradient, the bar of the forward pass.  bf16 inputs and
dh are exact in the oracle's float64.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import GATE, TOL, case, h_f64, rel_err, to_dev
from mlstm_sequence_amd import tfla

pytestmark = pytest.mark.gpu

SIG, SCAL, GLA = W.MLSTM_SIG, W.SCALAR, W.GLA
F32, BF = torch.float32, torch.bfloat16
NAMES = ["dq", "dk", "dv", "dig", "dfg"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def oracle_bwd(inp, dh, variant):
    return oracle.recurrent_bwd(W.as_f64(inp["q"]), W.as_f64(inp["k"]), W.as_f64(inp["v"]),
                                W.as_f64(inp["igate_pre"]), W.as_f64(inp["fgate_pre"]), W.as_f64(dh), variant)


def gpu_bwd(inp, dh, variant, L, workspace=False):
    """tfla_bwd on device copies; every output prefilled with NaN so each
    element must be written."""
    d = to_dev(inp)
    q, k, v = d["q"], d["k"], d["v"]
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    var = tfla.variant_of(GATE[variant], q.dtype)
    nan = float("nan")
    dq = torch.full_like(q, nan)
    dk = torch.full_like(k, nan)
    dv = torch.full_like(v, nan)
    dig = None if d["igate_pre"] is None else torch.full_like(d["igate_pre"], nan)
    dfg = torch.full_like(d["fgate_pre"], nan)
    ws, nws = None, 0
    if workspace:
        nws = tfla.tfla_bwd_workspace_bytes(B, H, T, dqk, dhv, L, var)
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda")
    tfla.tfla_bwd(q, k, v, d["igate_pre"], d["fgate_pre"], dh.cuda(), dq, dk, dv, dig, dfg,
                  B, H, T, dqk, dhv, L, var, ws, nws)
    torch.cuda.synchronize()
    return dq, dk, dv, dig, dfg


def check(got, ref, dtype, label):
    for name, g, r in zip(NAMES, got, ref):
        if r is None:
            assert g is None
            continue
        err = rel_err(h_f64(g), r)
        print(f"  {label} {name}: {err:.3e}", flush=True)
        assert err <= TOL[dtype], f"{label} {name}: {err:.3e}"


BWD_CASES = [
    # variant, dtype, B, H, T, dqk, dhv, L
    (SIG, F32, 1, 2, 256, 64, 64, 64),
    (SIG, F32, 2, 1, 300, 128, 128, 128),
    (SIG, F32, 1, 1, 200, 64, 128, 64),        # d_qk != d_hv
    (SIG, BF, 1, 2, 700, 256, 512, 256),       # the headline head shape, ragged tail
    (SIG, BF, 2, 2, 530, 128, 128, 64),
    (SIG, BF, 1, 1, 40, 128, 256, 128),        # one partial chunk: no state at all
    (SIG, BF, 1, 1, 1000, 256, 128, 512),      # d_qk > d_hv, long chunks
    (SIG, BF, 4, 4, 1024, 128, 128, 128),      # 128x128 state tiles
    (SIG, BF, 1, 1, 1500, 64, 256, 64),        # few heads: segmented state walks
    (SCAL, BF, 1, 3, 333, 128, 128, 64),
    (SCAL, F32, 1, 2, 129, 64, 128, 128),
    (SCAL, BF, 2, 2, 600, 256, 512, 128),
    (GLA, BF, 1, 2, 450, 256, 256, 64),        # per-channel gate: output-side decay in dq, dk
    (GLA, F32, 1, 2, 200, 64, 128, 128),
    (GLA, BF, 2, 1, 700, 128, 512, 256),       # 512-wide contraction, long chunks
    (GLA, BF, 1, 1, 40, 64, 64, 64),           # one partial chunk
    (GLA, BF, 1, 2, 600, 128, 256, 256),       # 8-wave dq, dk: products stored without the fp32 staging
]


@pytest.mark.parametrize("variant,dtype,B,H,T,dqk,dhv,L", BWD_CASES)
def test_backward_matches_oracle(variant, dtype, B, H, T, dqk, dhv, L):
    wl, inp = case(variant, B, H, T, dqk, dhv, dtype, seed=3 * T + dqk + variant)
    dh = W.upstream_grad(B, H, T, dhv, dtype, seed=T + 11)
    print(f"bwd {variant} {dtype} B{B} H{H} T{T} {dqk}x{dhv} L{L}", flush=True)
    got = gpu_bwd(inp, dh, variant, L)
    check(got, oracle_bwd(inp, dh, variant), dtype, "bwd")


@pytest.mark.parametrize("segments", ["1", "2", "5"])
@pytest.mark.parametrize("variant", [SIG, SCAL, GLA])
def test_backward_segmented_walk(variant, segments, set_knob):
    """Forced segment counts of both state walks (the reverse walk's first
    segment holds the partial last chunk)."""
    set_knob(tfla.KNOB_STATE_SEGMENTS, segments)
    B, H, T, dqk, dhv, L = 1, 2, 64 * 11 + 29, 64, 128, 64
    wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=77 + variant)
    dh = W.upstream_grad(B, H, T, dhv, BF, seed=78)
    print(f"bwd segments={segments} variant={variant}", flush=True)
    got = gpu_bwd(inp, dh, variant, L, workspace=True)
    check(got, oracle_bwd(inp, dh, variant), BF, f"P={segments}")


@pytest.mark.parametrize("variant,B,H,dqk,dhv,segments", [
    (SIG, 1, 4, 256, 512, "3"),     # combine in 16-byte pieces, both walks
    (SCAL, 1, 2, 256, 512, "5"),    # 8-byte pieces
    (GLA, 4, 8, 256, 64, "3"),      # 16-byte pieces, 16 key channels per workgroup
])
def test_backward_segmented_walk_wide_combine(variant, B, H, dqk, dhv, segments, set_knob):
    """Forced segments at shapes whose combine passes (the forward walk's
    and the reverse walk's) take 8- or 16-byte pieces per thread."""
    set_knob(tfla.KNOB_STATE_SEGMENTS, segments)
    T, L = 64 * 13 + 5, 64
    wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=91 + variant + H)
    dh = W.upstream_grad(B, H, T, dhv, BF, seed=92)
    print(f"bwd wide combine: variant={variant} B{B} H{H} {dqk}x{dhv} segments={segments}", flush=True)
    got = gpu_bwd(inp, dh, variant, L, workspace=True)
    check(got, oracle_bwd(inp, dh, variant), BF, f"P={segments}")


def test_backward_chunk_size_invariance():
    """The gradients do not depend on the chunk size beyond rounding."""
    B, H, T, dqk, dhv = 1, 2, 1100, 128, 256
    wl, inp = case(SIG, B, H, T, dqk, dhv, BF, seed=5)
    dh = W.upstream_grad(B, H, T, dhv, BF, seed=6)
    ref = oracle_bwd(inp, dh, SIG)
    for L in (64, 128, 256, 512, 1024):
        print(f"bwd L={L}", flush=True)
        check(gpu_bwd(inp, dh, SIG, L), ref, BF, f"L={L}")


def test_backward_extreme_gates():
    """Input gates of exactly 0 and 1 (pre-activation -inf / +inf), forget
    gates of 1 and 0 (the latter at the log floor: no gradient)."""
    B, H, T, dqk, dhv, L = 1, 1, 300, 64, 64, 64
    wl, inp = case(SIG, B, H, T, dqk, dhv, F32, seed=9)
    ig, fg = inp["igate_pre"].clone(), inp["fgate_pre"].clone()
    ig[0, 0, 10:20] = -float("inf")
    ig[0, 0, 30:40] = float("inf")
    fg[0, 0, 50:60] = float("inf")
    fg[0, 0, 100] = -float("inf")
    fg[0, 0, 150] = -200.0
    inp = dict(inp, igate_pre=ig, fgate_pre=fg)
    dh = W.upstream_grad(B, H, T, dhv, F32, seed=10)
    got = gpu_bwd(inp, dh, SIG, L)
    for g in got[:3]:
        assert torch.isfinite(g).all()
    check(got, oracle_bwd(inp, dh, SIG), F32, "extreme")


def test_backward_workspace_entry_matches_allocating_entry():
    B, H, T, dqk, dhv, L = 2, 2, 500, 128, 128, 128
    wl, inp = case(SIG, B, H, T, dqk, dhv, BF, seed=12)
    dh = W.upstream_grad(B, H, T, dhv, BF, seed=13)
    a = gpu_bwd(inp, dh, SIG, L, workspace=False)
    b = gpu_bwd(inp, dh, SIG, L, workspace=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_rejects_odd_widths():
    wl, inp = case(SIG, 1, 1, 64, 64, 192, BF, seed=1)
    d = to_dev(inp)
    dh = torch.zeros_like(d["v"])
    out = [torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])]
    with pytest.raises(RuntimeError, match="unsupported"):
        tfla.tfla_bwd(d["q"], d["k"], d["v"], d["igate_pre"], d["fgate_pre"], dh, *out,
                      torch.empty_like(d["igate_pre"]), torch.empty_like(d["fgate_pre"]),
                      1, 1, 64, 64, 192, 64, tfla.variant_of(tfla.MLSTM_SIG, BF))
    assert tfla.tfla_bwd_workspace_bytes(1, 1, 64, 64, 192, 64, tfla.variant_of(tfla.MLSTM_SIG, BF)) == 0


@pytest.mark.parametrize("variant,dtype,T,L,segments", [
    (SIG, BF, 1100, 128, None), (SCAL, F32, 333, 64, None), (GLA, BF, 530, 64, None), (SIG, BF, 64 * 11 + 29, 64, "3"),
])
def test_backward_reusing_forward_workspace(variant, dtype, T, L, segments, set_knob):
    """tfla_fwd_ws leaves its gate sums and states in the workspace; tfla_bwd
    with TFLA_BWD_REUSE_FWD on that workspace skips recomputing them and
    returns bitwise the gradients of the recomputing call."""
    if segments:
        set_knob(tfla.KNOB_STATE_SEGMENTS, segments)
    B, H, dqk, dhv = 1, 2, 64, 128
    wl, inp = case(variant, B, H, T, dqk, dhv, dtype, seed=T + variant)
    dh = W.upstream_grad(B, H, T, dhv, dtype, seed=T + 1)
    ref = gpu_bwd(inp, dh, variant, L, workspace=True)
    d = to_dev(inp)
    var = tfla.variant_of(GATE[variant], dtype)
    nws = tfla.tfla_bwd_workspace_bytes(B, H, T, dqk, dhv, L, var)
    assert nws >= tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, L, var)
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bit patterns until written
    h = torch.empty_like(d["v"])
    tfla.tfla_fwd_ws(d["q"], d["k"], d["v"], d["igate_pre"], d["fgate_pre"], h, B, H, T, dqk, dhv, L, var, ws, nws)
    out = [torch.full_like(d["q"], float("nan")), torch.full_like(d["k"], float("nan")),
           torch.full_like(d["v"], float("nan")),
           None if d["igate_pre"] is None else torch.full_like(d["igate_pre"], float("nan")),
           torch.full_like(d["fgate_pre"], float("nan"))]
    for _ in range(2):   # the backward leaves the forward's part of the workspace intact
        tfla.tfla_bwd(d["q"], d["k"], d["v"], d["igate_pre"], d["fgate_pre"], dh.cuda(), *out, B, H, T, dqk, dhv, L,
                      var | tfla.BWD_REUSE_FWD, ws, nws)
        torch.cuda.synchronize()
        for name, x, y in zip(NAMES, out, ref):
            if y is not None:
                assert torch.equal(x, y), name


@pytest.mark.parametrize("variant", [SIG, SCAL, GLA])
@pytest.mark.parametrize("T,L", [(1, 64), (64, 64), (65, 64), (257, 128), (1024, 1024)])
def test_backward_sequence_edges(variant, T, L):
    """One step, exactly one chunk, one step into a second chunk, a one-row
    tail past several chunks, one whole 1024-step chunk."""
    B, H, dqk, dhv = 1, 1, 64, 64
    wl, inp = case(variant, B, H, T, dqk, dhv, F32, seed=T * 3 + variant)
    dh = W.upstream_grad(B, H, T, dhv, F32, seed=T + 2)
    print(f"bwd edge variant={variant} T={T} L={L}", flush=True)
    check(gpu_bwd(inp, dh, variant, L), oracle_bwd(inp, dh, variant), F32, f"T={T}")


def test_backward_is_deterministic():
    """No atomics: two calls give bitwise the same gradients."""
    B, H, T, dqk, dhv, L = 2, 2, 700, 128, 256, 128
    wl, inp = case(SIG, B, H, T, dqk, dhv, BF, seed=21)
    dh = W.upstream_grad(B, H, T, dhv, BF, seed=22)
    a = gpu_bwd(inp, dh, SIG, L)
    b = gpu_bwd(inp, dh, SIG, L)
    for x, y in zip(a, b):
        assert torch.equal(x, y)

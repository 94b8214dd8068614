"""TFLA_STATES_FP32: the forward pass with the chunk states materialised in
fp32 instead of bf16 (bf16 I/O).  The intra-chunk kernel rounds the states
to bf16 (RNE) for its matrix cores either way, so with the state walk rounding
each state once, h must agree to the last bit and the bf16 states must be
exactly the RNE rounding of the fp32 ones; both paths must match the oracle.
A walk cut into segments fixes up the states it stored by default (bf16
states rounded twice: the stored part, then the sum); these bitwise checks
take the two-pass form of the segmented walk (test override), and the
fix-up's own test bounds the difference it makes."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import GATE, TOL, case, h_f64, oracle_forward, rel_err, to_dev
from mlstm_sequence_amd import tfla

pytestmark = pytest.mark.gpu

SIG, SCAL, GLA = W.MLSTM_SIG, W.SCALAR, W.GLA
BF = torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tfla.lib()


@pytest.fixture
def two_pass():
    """Segmented state walks in their two-pass form (each state rounded once)."""
    with tfla.knob(tfla.KNOB_STATE_REWALK, 1):
        yield


def run_fwd(d, variant, L, flags=0):
    q, v = d["q"], d["v"]
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    h = torch.full((B, H, T, dhv), float("nan"), dtype=q.dtype, device=q.device)
    var = tfla.variant_of(GATE[variant], q.dtype) | flags
    tfla.tfla_fwd(q, d["k"], v, d["igate_pre"], d["fgate_pre"], h, B, H, T, dqk, dhv, L, var)
    torch.cuda.synchronize()
    return h


CASES = [
    # variant, B, H, T, dqk, dhv, L
    (SIG, 1, 2, 700, 256, 512, 256),
    (SIG, 2, 2, 600, 256, 512, 64),
    (SIG, 1, 2, 1100, 64, 64, 512),
    (SIG, 1, 1, 2100, 128, 256, 1024),
    (SIG, 1, 2, 64 * 40, 128, 128, 64),     # a chain long enough for the segmented state walk
    (SCAL, 2, 4, 500, 128, 128, 64),
    (SCAL, 1, 2, 900, 256, 320, 256),
    (GLA, 2, 2, 400, 256, 512, 64),
    (GLA, 1, 1, 600, 128, 256, 256),
]


@pytest.mark.parametrize("variant,B,H,T,dqk,dhv,L", CASES)
def test_fp32_states_give_the_same_h(two_pass, variant, B, H, T, dqk, dhv, L):
    print(f"fp32 states: variant {variant} B{B} H{H} T{T} {dqk}x{dhv} L{L}", flush=True)
    wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=31 * T + dqk)
    d = to_dev(inp)
    h16 = run_fwd(d, variant, L)
    h32 = run_fwd(d, variant, L, tfla.STATES_FP32)
    assert torch.equal(h16, h32)
    assert rel_err(h_f64(h32), oracle_forward(inp, variant)) <= TOL[BF]


@pytest.mark.parametrize("variant,dqk,dhv,T,L", [
    (SIG, 256, 512, 700, 128), (SIG, 128, 192, 640, 64), (SCAL, 128, 128, 520, 64), (GLA, 256, 128, 512, 64),
])
def test_bf16_states_are_the_rounded_fp32_states(two_pass, variant, dqk, dhv, T, L):
    wl, inp = case(variant, 1, 2, T, dqk, dhv, BF, seed=dqk + 3 * T)
    d = to_dev(inp)
    nc = -(-T // L)
    var = tfla.variant_of(GATE[variant], BF)
    st16 = torch.full((1, 2, nc - 1, dhv, dqk), float("nan"), device="cuda", dtype=BF)
    st32 = torch.full((1, 2, nc - 1, dhv, dqk), float("nan"), device="cuda", dtype=torch.float32)
    tfla.tfla_dbg_states(d["k"], d["v"], d["igate_pre"], d["fgate_pre"], st16, 1, 2, T, dqk, dhv, L, var)
    tfla.tfla_dbg_states(d["k"], d["v"], d["igate_pre"], d["fgate_pre"], st32, 1, 2, T, dqk, dhv, L,
                         var | tfla.STATES_FP32)
    torch.cuda.synchronize()
    assert torch.equal(st16, st32.to(BF))
    _, st_ref = oracle_forward(inp, variant, L=L)
    assert rel_err(st32.cpu().double().numpy().swapaxes(-1, -2), st_ref[:, :, :nc - 1]) <= TOL[BF]


@pytest.mark.parametrize("variant", [SIG, SCAL, GLA])
def test_fp32_states_with_initial_and_final_state(two_pass, variant):
    B, H, T, dqk, dhv, L = 1, 2, 650, 128, 256, 128
    wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=77)
    d = to_dev(inp)
    c0 = W.initial_state(B, H, dqk, dhv, seed=5, std=1.5).cuda()
    var = tfla.variant_of(GATE[variant], BF)
    outs = []
    for flags in (0, tfla.STATES_FP32):
        h = torch.full((B, H, T, dhv), float("nan"), dtype=BF, device="cuda")
        cf = torch.full((B, H, dqk, dhv), float("nan"), device="cuda")
        tfla.tfla_fwd_state(d["q"], d["k"], d["v"], d["igate_pre"], d["fgate_pre"], c0, h, cf, B, H, T, dqk, dhv,
                            L, var | flags)
        torch.cuda.synchronize()
        outs.append((h, cf))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def test_fp32_states_full_size_headline_workload(two_pass):
    """Workload 3 at L = 256: the launch configuration the bench times."""
    wl = W.WORKLOADS[3]
    inp = W.make_inputs(wl)
    d = to_dev(inp)
    h16 = run_fwd(d, wl.variant, 256)
    h32 = run_fwd(d, wl.variant, 256, tfla.STATES_FP32)
    assert torch.equal(h16, h32)


@pytest.mark.parametrize("variant,B,H,T,dqk,dhv,L", [
    (SIG, 2, 2, 600, 256, 512, 64), (SIG, 1, 2, 64 * 40, 128, 128, 64), (GLA, 2, 2, 400, 256, 512, 64),
])
def test_fixup_walk_with_fp32_states(variant, B, H, T, dqk, dhv, L):
    """The default segmented walk (fix-up of the stored states): the bf16
    states differ from the RNE rounding of the fp32 states by at most a unit
    of bf16 of the largest state (the stored part is rounded before the start
    state is added), h of the two by at most two, and both match the oracle."""
    wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=31 * T + dqk)
    d = to_dev(inp)
    print(f"fix-up walk, fp32 states: variant {variant} B{B} H{H} T{T} {dqk}x{dhv} L{L}", flush=True)
    h16 = run_fwd(d, variant, L)
    h32 = run_fwd(d, variant, L, tfla.STATES_FP32)
    ref = oracle_forward(inp, variant)
    assert rel_err(h_f64(h16), ref) <= TOL[BF]
    assert rel_err(h_f64(h32), ref) <= TOL[BF]
    assert rel_err(h_f64(h16), h_f64(h32)) <= 2 * 2.0 ** -8
    nc = -(-T // L)
    var = tfla.variant_of(GATE[variant], BF)
    st16 = torch.full((B, H, nc - 1, dhv, dqk), float("nan"), device="cuda", dtype=BF)
    st32 = torch.full((B, H, nc - 1, dhv, dqk), float("nan"), device="cuda", dtype=torch.float32)
    tfla.tfla_dbg_states(d["k"], d["v"], d["igate_pre"], d["fgate_pre"], st16, B, H, T, dqk, dhv, L, var)
    tfla.tfla_dbg_states(d["k"], d["v"], d["igate_pre"], d["fgate_pre"], st32, B, H, T, dqk, dhv, L,
                         var | tfla.STATES_FP32)
    torch.cuda.synchronize()
    # largest difference against the largest state: a unit of bf16 at most
    assert rel_err(st16.double().cpu().numpy(), st32.to(BF).double().cpu().numpy()) <= 2.0 ** -7

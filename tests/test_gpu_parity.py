"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Tolerance: max|h_gpu - h_oracle| / max|h_oracle| <= 1e-4 for fp32 I/O and
<= 2e-2 for bf16 I/O (fp32 accumulation), computed in double.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import GATE, TOL, case, gpu_forward, h_f64, oracle_forward, rel_err
from mlstm_sequence_amd import tfla

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SIG, SCAL, GLA = W.MLSTM_SIG, W.SCALAR, W.GLA
F32, BF = torch.float32, torch.bfloat16


# ---------------------------------------------------------------- gate kernel
@pytest.mark.parametrize("variant", [SIG, SCAL, GLA])
@pytest.mark.parametrize("T,L", [(1, 64), (200, 64), (333, 128), (1500, 256)])
def test_gate_prefix_sums(variant, T, L):
    wl, inp = case(variant, 2, 3, T, 64, 64, BF, seed=T + variant)
    a_ref, li_ref, g_ref = oracle.log_gates(W.as_f64(inp["igate_pre"]), W.as_f64(inp["fgate_pre"]), variant,
                                            2, 3, T, 64, L)
    nc = -(-T // L)
    wdt = 64 if variant == GLA else 1
    a = torch.full((2, 3, T * wdt), float("nan"), device="cuda")
    li = torch.full((2, 3, T), float("nan"), device="cuda")
    g = torch.full((2, 3, nc * wdt), float("nan"), device="cuda")
    ig = None if inp["igate_pre"] is None else inp["igate_pre"].cuda()
    tfla.tfla_dbg_gates(ig, inp["fgate_pre"].cuda(), a, li, g, 2, 3, T, 64, L,
                        tfla.variant_of(GATE[variant], BF))
    torch.cuda.synchronize()
    assert rel_err(a.cpu().numpy().reshape(a_ref.shape), a_ref) <= 1e-5
    assert rel_err(g.cpu().numpy().reshape(g_ref.shape), g_ref) <= 1e-5
    assert rel_err(li.cpu().numpy(), li_ref) <= 1e-6


@pytest.mark.parametrize("dqk", [64, 128, 256])
@pytest.mark.parametrize("T,L", [(1, 64), (97, 64), (700, 128), (900, 256), (1500, 512), (2100, 1024)])
def test_per_channel_gate_prefix_sums(dqk, T, L):
    """The per-channel gate kernel (16 steps x 4 channels per thread, segment
    totals through LDS, a carry across passes when the chunk is longer than
    one pass) at every d_qk and chunk size, ragged last chunks included."""
    print(f"per-channel gate sums: d_qk {dqk} T {T} L {L}", flush=True)
    wl, inp = case(GLA, 1, 2, T, dqk, 64, BF, seed=T + dqk + L)
    a_ref, _, g_ref = oracle.log_gates(None, W.as_f64(inp["fgate_pre"]), GLA, 1, 2, T, dqk, L)
    nc = -(-T // L)
    a = torch.full((1, 2, T * dqk), float("nan"), device="cuda")
    li = torch.full((1, 2, T), float("nan"), device="cuda")
    g = torch.full((1, 2, nc * dqk), float("nan"), device="cuda")
    tfla.tfla_dbg_gates(None, inp["fgate_pre"].cuda(), a, li, g, 1, 2, T, dqk, L, tfla.variant_of(tfla.GLA_KEY, BF))
    torch.cuda.synchronize()
    assert rel_err(a.cpu().numpy().reshape(a_ref.shape), a_ref) <= 1e-5
    assert rel_err(g.cpu().numpy().reshape(g_ref.shape), g_ref) <= 1e-5


# ---------------------------------------------------------------- state kernel
@pytest.mark.parametrize("variant,dtype,dqk,dhv,T,L", [
    (SIG, F32, 64, 64, 256, 64), (SIG, BF, 256, 512, 700, 128), (SIG, BF, 128, 192, 640, 64),
    (SCAL, BF, 128, 128, 520, 64), (SCAL, F32, 128, 64, 300, 128),
    (GLA, BF, 256, 128, 512, 64), (GLA, F32, 64, 128, 390, 128),
])
def test_states(variant, dtype, dqk, dhv, T, L):
    wl, inp = case(variant, 1, 2, T, dqk, dhv, dtype, seed=dqk + T)
    _, st_ref = oracle_forward(inp, variant, L=L)
    nc = -(-T // L)
    st = torch.full((1, 2, nc - 1, dhv, dqk), float("nan"), device="cuda", dtype=dtype)   # I/O type
    ig = None if inp["igate_pre"] is None else inp["igate_pre"].cuda()
    tfla.tfla_dbg_states(inp["k"].cuda(), inp["v"].cuda(), ig, inp["fgate_pre"].cuda(), st, 1, 2, T, dqk, dhv, L,
                         tfla.variant_of(GATE[variant], dtype))
    torch.cuda.synchronize()
    got = st.cpu().double().numpy().swapaxes(-1, -2)
    tol = 1e-5 if dtype == F32 else 2e-2
    assert rel_err(got, st_ref[:, :, :nc - 1]) <= tol


# ---------------------------------------------------------------- end to end, small
SMALL = [
    # variant, dtype, B, H, T, dqk, dhv, L
    (SIG, F32, 1, 1, 256, 64, 64, 64),
    (SIG, F32, 2, 2, 333, 128, 128, 64),
    (SIG, F32, 1, 2, 450, 64, 192, 128),
    (SIG, BF, 2, 2, 600, 256, 512, 64),
    (SIG, BF, 1, 2, 777, 256, 512, 128),
    (SIG, BF, 1, 2, 700, 256, 512, 256),
    (SIG, BF, 1, 3, 530, 128, 128, 128),
    (SIG, BF, 2, 1, 1100, 64, 64, 512),
    (SIG, BF, 1, 1, 2100, 128, 256, 1024),
    (SCAL, BF, 2, 4, 500, 128, 128, 64),
    (SCAL, F32, 1, 3, 300, 64, 128, 128),
    (SCAL, BF, 1, 2, 900, 256, 320, 256),
    (GLA, BF, 2, 2, 400, 256, 512, 64),
    (GLA, BF, 1, 2, 300, 64, 128, 128),
    (GLA, F32, 1, 2, 270, 128, 64, 64),
    (GLA, BF, 1, 1, 600, 128, 256, 256),
]


@pytest.mark.parametrize("variant,dtype,B,H,T,dqk,dhv,L", SMALL)
def test_parity_small(variant, dtype, B, H, T, dqk, dhv, L):
    wl, inp = case(variant, B, H, T, dqk, dhv, dtype, seed=17 * T + dqk)
    ref = oracle_forward(inp, variant)
    h = gpu_forward(inp, variant, L)
    assert rel_err(h_f64(h), ref) <= TOL[dtype]


@pytest.mark.parametrize("variant,dtype", [(SIG, BF), (SIG, F32), (SCAL, BF), (GLA, BF)])
@pytest.mark.parametrize("T,L", [(1, 64), (37, 64), (64, 64), (65, 64), (129, 128), (255, 256)])
def test_edge_lengths(variant, dtype, T, L):
    """One step, a partial single chunk, exactly one chunk, one step into a
    second chunk."""
    wl, inp = case(variant, 1, 1, T, 64, 64, dtype, seed=T)
    ref = oracle_forward(inp, variant)
    h = gpu_forward(inp, variant, L)
    assert rel_err(h_f64(h), ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [F32, BF])
def test_degenerate_gates(dtype):
    """Gates of exactly 1 (pre-activation +inf), exactly 0 (-inf) and a zero
    input gate, mixed into one sequence."""
    wl, inp = case(SIG, 1, 2, 300, 64, 128, dtype, seed=5)
    fg, ig = inp["fgate_pre"].clone(), inp["igate_pre"].clone()
    fg[0, 0, 10:40] = float("inf")
    fg[0, 0, 70] = float("-inf")
    fg[0, 1, 130:135] = float("-inf")
    ig[0, 0, 50:60] = float("-inf")
    ig[0, 1, 200:] = float("inf")
    inp.update(fgate_pre=fg, igate_pre=ig)
    ref = oracle_forward(inp, SIG)
    h = gpu_forward(inp, SIG, 64)
    assert rel_err(h_f64(h), ref) <= TOL[dtype]


def test_no_decay_is_causal_linear_attention():
    """Scalar decay with logit +inf: gamma = 1, causal linear attention."""
    wl, inp = case(SCAL, 1, 2, 400, 128, 128, BF, seed=8)
    inp["fgate_pre"] = torch.full((2,), float("inf"))
    ref = oracle_forward(inp, SCAL)
    h = gpu_forward(inp, SCAL, 128)
    assert rel_err(h_f64(h), ref) <= TOL[BF]


def test_channel_constant_gla_matches_scalar_gate():
    """GLA with the same gate on every channel equals the mLSTMsig path with
    i = 1 and f = exp(logsigmoid(x)/16)."""
    wl, inp = case(GLA, 1, 2, 500, 128, 128, BF, seed=12)
    x = inp["fgate_pre"][..., :1].expand(-1, -1, -1, 128).contiguous()
    inp["fgate_pre"] = x
    h_gla = h_f64(gpu_forward(inp, GLA, 64))
    xd = x[..., 0].double()
    lf = (torch.minimum(xd, torch.zeros_like(xd)) - torch.log1p(torch.exp(-xd.abs()))) / 16
    fpre = (lf - torch.log1p(-torch.exp(lf))).float()   # logit of f
    sig = dict(inp, fgate_pre=fpre, igate_pre=torch.full((1, 2, 500), float("inf")))
    h_sig = h_f64(gpu_forward(sig, SIG, 64))
    assert rel_err(h_gla, h_sig) <= 2e-2


# ---------------------------------------------------------------- properties
def test_deterministic_and_ws_equals_alloc():
    wl, inp = case(SIG, 2, 2, 700, 256, 512, BF, seed=3)
    h1 = gpu_forward(inp, SIG, 128)
    h2 = gpu_forward(inp, SIG, 128)
    h3 = gpu_forward(inp, SIG, 128, workspace=True)
    assert torch.equal(h1, h2) and torch.equal(h1, h3)


@pytest.mark.parametrize("variant", [SIG, GLA])
def test_causality_bitwise(variant):
    wl, inp = case(variant, 1, 2, 640, 128, 128, BF, seed=4)
    h = gpu_forward(inp, variant, 128)
    t0 = 300
    inp2 = dict(inp)
    for n in ("q", "k", "v"):
        x = inp[n].clone()
        x[:, :, t0:] = (x[:, :, t0:].float() * -2.0 + 1.0).to(x.dtype)
        inp2[n] = x
    h2 = gpu_forward(inp2, variant, 128)
    assert torch.equal(h[:, :, :t0], h2[:, :, :t0])
    assert not torch.equal(h[:, :, t0:], h2[:, :, t0:])


def test_chunk_size_invariance():
    wl, inp = case(SIG, 1, 2, 1024, 128, 256, BF, seed=6)
    ref = oracle_forward(inp, SIG)
    outs = {L: h_f64(gpu_forward(inp, SIG, L)) for L in (64, 128, 256, 512, 1024)}
    for L, h in outs.items():
        assert rel_err(h, ref) <= TOL[BF], L
        assert rel_err(h, outs[64]) <= TOL[BF], L

"""tfla_bwd_state (the backward pass from an initial state, with a gradient
on the final state) through the C ABI against the oracle's
recurrent_bwd_state, element by element; tolerances of the forward pass
(max|d|/max|ref| <= 1e-4 fp32, <= 2e-2 bf16) on every gradient and dL/dC_0."""
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
NAMES = ["dq", "dk", "dv", "dig", "dfg", "dc0"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def states(B, H, dqk, dhv, seed, with_c0, with_g):
    c0 = W.initial_state(B, H, dqk, dhv, seed=seed, std=1.5) if with_c0 else None
    g = W.initial_state(B, H, dqk, dhv, seed=seed + 1, std=0.5) if with_g else None
    return c0, g


def gpu_bwd_state(inp, dh, variant, L, c0=None, dcT=None, want_dc0=True, workspace=True, in_place=None):
    d = to_dev(inp)
    q, k, v = d["q"], d["k"], d["v"]
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    var = tfla.variant_of(GATE[variant], q.dtype)
    nan = float("nan")
    out = [torch.full_like(q, nan), torch.full_like(k, nan), torch.full_like(v, nan),
           None if d["igate_pre"] is None else torch.full_like(d["igate_pre"], nan),
           torch.full_like(d["fgate_pre"], nan)]
    c0d = None if c0 is None else c0.cuda()
    gd = None if dcT is None else dcT.cuda()
    if in_place == "c0":
        dc0 = c0d
    elif in_place == "dc_final":
        dc0 = gd
    else:
        dc0 = torch.full((B, H, dqk, dhv), nan, device="cuda") if want_dc0 else None
    ws, nws = None, 0
    if workspace:
        nws = tfla.tfla_bwd_state_workspace_bytes(B, H, T, dqk, dhv, L, var)
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda")
    tfla.tfla_bwd_state(q, k, v, d["igate_pre"], d["fgate_pre"], c0d, dh.cuda(), gd, *out, dc0,
                        B, H, T, dqk, dhv, L, var, ws, nws)
    torch.cuda.synchronize()
    return out + [dc0]


def oracle_state(inp, dh, variant, c0, dcT):
    return oracle.recurrent_bwd_state(W.as_f64(inp["q"]), W.as_f64(inp["k"]), W.as_f64(inp["v"]),
                                      W.as_f64(inp["igate_pre"]), W.as_f64(inp["fgate_pre"]), W.as_f64(dh), variant,
                                      c0=None if c0 is None else c0.double().numpy(),
                                      dcT=None if dcT is None else dcT.double().numpy())


def check(got, ref, dtype, label):
    for name, g, r in zip(NAMES, got, ref):
        if r is None or g is None:
            continue
        err = rel_err(h_f64(g), r)
        print(f"  {label} {name}: {err:.3e}", flush=True)
        assert err <= TOL[dtype], f"{label} {name}: {err:.3e}"


CASES = [
    # variant, dtype, B, H, T, dqk, dhv, L
    (SIG, F32, 1, 2, 300, 64, 64, 64),
    (SIG, BF, 1, 2, 530, 128, 256, 128),
    (SIG, BF, 2, 1, 700, 256, 512, 256),
    (SCAL, BF, 1, 3, 333, 128, 128, 64),
    (SCAL, F32, 1, 2, 200, 64, 128, 128),
    (GLA, BF, 1, 2, 450, 128, 256, 64),
    (GLA, F32, 1, 1, 150, 64, 64, 64),
]


@pytest.mark.parametrize("with_c0,with_g", [(True, True), (True, False), (False, True), (False, False)])
@pytest.mark.parametrize("variant,dtype,B,H,T,dqk,dhv,L", CASES)
def test_state_backward_matches_oracle(variant, dtype, B, H, T, dqk, dhv, L, with_c0, with_g):
    wl, inp = case(variant, B, H, T, dqk, dhv, dtype, seed=5 * T + dqk + variant)
    dh = W.upstream_grad(B, H, T, dhv, dtype, seed=T + 3)
    c0, g = states(B, H, dqk, dhv, T + 4, with_c0, with_g)
    print(f"bwd_state {variant} {dtype} T{T} {dqk}x{dhv} L{L} c0={with_c0} dcT={with_g}", flush=True)
    got = gpu_bwd_state(inp, dh, variant, L, c0=c0, dcT=g)
    check(got, oracle_state(inp, dh, variant, c0, g), dtype, "state")


@pytest.mark.parametrize("segments", ["2", "5"])
@pytest.mark.parametrize("variant", [SIG, SCAL, GLA])
def test_state_backward_segmented_walks(variant, segments, set_knob):
    set_knob(tfla.KNOB_STATE_SEGMENTS, segments)
    B, H, T, dqk, dhv, L = 1, 2, 64 * 11 + 29, 64, 128, 64
    wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=31 + variant)
    dh = W.upstream_grad(B, H, T, dhv, BF, seed=32)
    c0, g = states(B, H, dqk, dhv, 33, True, True)
    check(gpu_bwd_state(inp, dh, variant, L, c0=c0, dcT=g), oracle_state(inp, dh, variant, c0, g), BF, f"P={segments}")


@pytest.mark.parametrize("variant", [SIG, SCAL, GLA])
@pytest.mark.parametrize("T,L", [(1, 64), (40, 64), (64, 64), (65, 64)])
def test_state_backward_short_sequences(variant, T, L):
    B, H, dqk, dhv = 1, 1, 64, 64
    wl, inp = case(variant, B, H, T, dqk, dhv, F32, seed=T + 40 + variant)
    dh = W.upstream_grad(B, H, T, dhv, F32, seed=T + 41)
    c0, g = states(B, H, dqk, dhv, T + 42, True, True)
    check(gpu_bwd_state(inp, dh, variant, L, c0=c0, dcT=g, workspace=False), oracle_state(inp, dh, variant, c0, g),
          F32, f"T={T}")


@pytest.mark.parametrize("which", ["c0", "dc_final"])
def test_state_backward_in_place(which):
    B, H, T, dqk, dhv, L = 1, 2, 300, 64, 128, 64
    wl, inp = case(SIG, B, H, T, dqk, dhv, F32, seed=50)
    dh = W.upstream_grad(B, H, T, dhv, F32, seed=51)
    c0, g = states(B, H, dqk, dhv, 52, True, True)
    ref = oracle_state(inp, dh, SIG, c0, g)
    got = gpu_bwd_state(inp, dh, SIG, L, c0=c0.clone(), dcT=g.clone(), in_place=which)
    check(got, ref, F32, f"in place of {which}")


def test_state_backward_without_states_equals_tfla_bwd():
    from test_gpu_bwd import gpu_bwd
    B, H, T, dqk, dhv, L = 2, 2, 500, 128, 128, 128
    for variant in (SIG, SCAL, GLA):
        wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=60 + variant)
        dh = W.upstream_grad(B, H, T, dhv, BF, seed=61)
        a = gpu_bwd(inp, dh, variant, L, workspace=True)
        b = gpu_bwd_state(inp, dh, variant, L, want_dc0=False)
        for x, y in zip(a, b[:5]):
            if x is not None:
                assert torch.equal(x, y), variant


@pytest.mark.parametrize("variant", [SIG, GLA])
def test_state_backward_chains_a_split_sequence(variant):
    """Two segments: the forward of the second starts from the first's final
    state; the backward of the second hands dL/dC_0 to the first as its
    final-state gradient.  The joined gradients match tfla_bwd of the whole
    sequence (and the oracle)."""
    from test_gpu_bwd import gpu_bwd, oracle_bwd
    B, H, T, dqk, dhv, L, m = 1, 2, 1000, 128, 128, 128, 384
    wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=70 + variant)
    dh = W.upstream_grad(B, H, T, dhv, BF, seed=71)
    cut = lambda x, a, b: None if x is None else x[:, :, a:b].contiguous()
    first = {n: cut(t, 0, m) for n, t in inp.items()}
    second = {n: cut(t, m, T) for n, t in inp.items()}
    d1 = to_dev(first)
    var = tfla.variant_of(GATE[variant], BF)
    c_mid = torch.empty((B, H, dqk, dhv), device="cuda")
    h1 = torch.empty_like(d1["v"])
    tfla.tfla_fwd_state(d1["q"], d1["k"], d1["v"], d1["igate_pre"], d1["fgate_pre"], None, h1, c_mid,
                        B, H, m, dqk, dhv, L, var)
    torch.cuda.synchronize()
    g2 = gpu_bwd_state(second, cut(dh, m, T), variant, L, c0=c_mid.cpu())
    g1 = gpu_bwd_state(first, cut(dh, 0, m), variant, L, dcT=g2[5].cpu())
    ref = oracle_bwd(inp, dh, variant)
    for i, name in enumerate(NAMES[:5]):
        if ref[i] is None:
            continue
        joined = np.concatenate([h_f64(g1[i]), h_f64(g2[i])], axis=2)
        err = rel_err(joined, ref[i])
        print(f"  chained {name}: {err:.3e}", flush=True)
        assert err <= TOL[BF], name

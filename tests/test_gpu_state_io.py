"""Initial / final state I/O and the fused recurrent kernel, through the C
ABI, against the oracle's recurrence from a given initial state.

Tolerances as for the forward pass: max|d|/max|ref| <= 1e-4 (fp32 I/O) and
<= 2e-2 (bf16 I/O) on h; states <= 1e-5 (fp32) and <= 2e-2 (bf16).
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
STOL = {F32: 1e-5, BF: 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def oracle_state(inp, variant, c0):
    return oracle.recurrent_fwd_state(W.as_f64(inp["q"]), W.as_f64(inp["k"]), W.as_f64(inp["v"]),
                                      W.as_f64(inp["igate_pre"]), W.as_f64(inp["fgate_pre"]), variant,
                                      c0=None if c0 is None else c0.double().numpy())


def run_state(d, variant, L, c0=None, want_final=True, in_place=False, workspace=False):
    """tfla_fwd_state on device inputs `d`; h prefilled with NaN."""
    q, v = d["q"], d["v"]
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    var = tfla.variant_of(GATE[variant], q.dtype)
    h = torch.full((B, H, T, dhv), float("nan"), dtype=q.dtype, device="cuda")
    c0d = None if c0 is None else c0.cuda()   # a device tensor is used as it is
    if in_place:
        cf = c0d
    else:
        cf = torch.full((B, H, dqk, dhv), float("nan"), device="cuda") if want_final else None
    ws, nws = None, 0
    if workspace:
        nws = tfla.tfla_state_workspace_bytes(B, H, T, dqk, dhv, L, var)
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda")
    tfla.tfla_fwd_state(q, d["k"], v, d["igate_pre"], d["fgate_pre"], c0d, h, cf, B, H, T, dqk, dhv, L, var,
                        ws, nws)
    torch.cuda.synchronize()
    return h, cf


STATE_CASES = [
    # variant, dtype, B, H, T, dqk, dhv, L
    (SIG, F32, 1, 2, 256, 64, 64, 64),
    (SIG, F32, 2, 1, 300, 128, 128, 128),
    (SIG, BF, 1, 2, 700, 256, 512, 256),
    (SIG, BF, 2, 2, 530, 128, 128, 64),
    (SIG, BF, 1, 1, 40, 128, 256, 128),        # one partial chunk
    (SIG, BF, 4, 4, 1024, 128, 128, 128),      # 128x128 state tiles
    (SCAL, BF, 1, 3, 333, 128, 128, 64),
    (SCAL, F32, 1, 2, 129, 64, 192, 128),
    (GLA, BF, 1, 2, 450, 256, 256, 64),
    (GLA, F32, 1, 2, 200, 64, 128, 128),
]


@pytest.mark.parametrize("variant,dtype,B,H,T,dqk,dhv,L", STATE_CASES)
@pytest.mark.parametrize("with_c0", [False, True])
def test_initial_and_final_state(variant, dtype, B, H, T, dqk, dhv, L, with_c0):
    wl, inp = case(variant, B, H, T, dqk, dhv, dtype, seed=T + 7 * dqk + variant)
    c0 = W.initial_state(B, H, dqk, dhv, seed=T + dhv, std=2.0) if with_c0 else None
    print(f"state I/O {variant} {dtype} B{B} H{H} T{T} {dqk}x{dhv} L{L} c0={with_c0}", flush=True)
    h, cf = run_state(to_dev(inp), variant, L, c0=c0)
    h_ref, c_ref = oracle_state(inp, variant, c0)
    assert rel_err(h_f64(h), h_ref) <= TOL[dtype]
    assert rel_err(cf.cpu().double().numpy(), c_ref) <= STOL[dtype]


@pytest.mark.parametrize("variant,dtype,B,H,T,dqk,dhv,L", [STATE_CASES[2], STATE_CASES[5], STATE_CASES[8]])
def test_state_in_place_and_workspace(variant, dtype, B, H, T, dqk, dhv, L):
    """c_final == c0 (in place) and a caller-owned workspace give the same
    bits as separate buffers and the library's own workspace."""
    wl, inp = case(variant, B, H, T, dqk, dhv, dtype, seed=99 + T)
    c0 = W.initial_state(B, H, dqk, dhv, seed=5, std=1.0)
    d = to_dev(inp)
    h1, cf1 = run_state(d, variant, L, c0=c0)
    h2, cf2 = run_state(d, variant, L, c0=c0, in_place=True, workspace=True)
    assert torch.equal(h1, h2)
    assert torch.equal(cf1, cf2)


@pytest.mark.parametrize("variant,dtype,B,H,T,dqk,dhv,L", STATE_CASES[:4] + STATE_CASES[6:])
def test_no_state_equals_forward(variant, dtype, B, H, T, dqk, dhv, L):
    """Without c0 and c_final the call is tfla_fwd, bit for bit."""
    wl, inp = case(variant, B, H, T, dqk, dhv, dtype, seed=3 + T)
    d = to_dev(inp)
    h1, _ = run_state(d, variant, L, want_final=False)
    h2 = tfla.forward(d["q"], d["k"], d["v"], d["igate_pre"], d["fgate_pre"], GATE[variant], L)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)


def part(inp, variant, lo, hi):
    out = {}
    for key, t in inp.items():
        if t is None or (variant == SCAL and key == "fgate_pre"):
            out[key] = t
        else:
            out[key] = t[:, :, lo:hi].contiguous()
    return out


@pytest.mark.parametrize("variant,dtype,dqk,dhv,L,cuts", [
    (SIG, BF, 128, 128, 64, [0, 256, 600, 1000]),
    (SIG, F32, 64, 128, 128, [0, 100, 101, 500]),
    (SCAL, BF, 128, 256, 128, [0, 384, 700]),
    (GLA, BF, 256, 128, 64, [0, 130, 512]),
])
def test_sequence_split_into_calls(variant, dtype, dqk, dhv, L, cuts):
    """Calls over consecutive segments, each starting from the previous
    call's final state, reproduce the whole sequence."""
    T = cuts[-1]
    wl, inp = case(variant, 1, 2, T, dqk, dhv, dtype, seed=31 + T)
    h_ref, c_ref = oracle_state(inp, variant, None)
    state = torch.zeros((1, 2, dqk, dhv), device="cuda")
    outs = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        h, state = run_state(to_dev(part(inp, variant, lo, hi)), variant, L, c0=state)
        outs.append(h_f64(h))
    assert rel_err(np.concatenate(outs, axis=2), h_ref) <= TOL[dtype]
    assert rel_err(state.cpu().double().numpy(), c_ref) <= STOL[dtype]


# ---------------------------------------------------------------- recurrent kernel
def run_recurrent(d, variant, state):
    q, v = d["q"], d["v"]
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    h = torch.full((B, H, T, dhv), float("nan"), dtype=q.dtype, device="cuda")
    tfla.tfla_fwd_recurrent(q, d["k"], v, d["igate_pre"], d["fgate_pre"], state, h, B, H, T, dqk, dhv,
                            tfla.variant_of(GATE[variant], q.dtype))
    torch.cuda.synchronize()
    return h


@pytest.mark.parametrize("variant,dtype,B,H,dqk,dhv", [
    (SIG, F32, 1, 2, 64, 64), (SIG, BF, 2, 2, 128, 192), (SIG, BF, 1, 2, 256, 512),
    (SCAL, BF, 1, 3, 128, 128), (SCAL, F32, 2, 1, 64, 256), (GLA, BF, 1, 2, 256, 128), (GLA, F32, 1, 2, 128, 64),
])
@pytest.mark.parametrize("T", [1, 5, 16, 37])
def test_recurrent_kernel(variant, dtype, B, H, dqk, dhv, T):
    wl, inp = case(variant, B, H, T, dqk, dhv, dtype, seed=11 * T + dqk)
    c0 = W.initial_state(B, H, dqk, dhv, seed=T, std=2.0)
    state = c0.cuda()
    h = run_recurrent(to_dev(inp), variant, state)
    h_ref, c_ref = oracle_state(inp, variant, c0)
    assert rel_err(h_f64(h), h_ref) <= TOL[dtype]
    assert rel_err(state.cpu().double().numpy(), c_ref) <= 1e-5


@pytest.mark.parametrize("variant", [SIG, SCAL, GLA])
def test_prefill_then_decode(variant):
    """A chunkwise prefill that returns its final state, then single decode
    steps with the recurrent kernel, equals one recurrence over all steps."""
    T0, n = 300, 6
    wl, inp = case(variant, 1, 2, T0 + n, 128, 128, BF, seed=123 + variant)
    h_ref, c_ref = oracle_state(inp, variant, None)
    h0, state = run_state(to_dev(part(inp, variant, 0, T0)), variant, 128)
    outs = [h_f64(h0)]
    for t in range(T0, T0 + n):
        outs.append(h_f64(run_recurrent(to_dev(part(inp, variant, t, t + 1)), variant, state)))
    assert rel_err(np.concatenate(outs, axis=2), h_ref) <= TOL[BF]
    assert rel_err(state.cpu().double().numpy(), c_ref) <= STOL[BF]


def test_long_context_split_in_two():
    """The long-context workload (B=1, H=8, T=65536, d=128, bf16, L=256) as
    two calls of 32768 steps chained through the state, against the oracle
    on two sampled heads over the whole sequence."""
    wl = W.WORKLOADS[5]
    inp = W.make_inputs(wl)
    heads = [(0, 0), (0, 5)]
    h_ref, c_ref = oracle_state(W.head_slice(inp, wl.variant, heads), wl.variant, None)
    half = wl.T // 2
    h1, st = run_state(to_dev(part(inp, wl.variant, 0, half)), wl.variant, 256)
    h2, st = run_state(to_dev(part(inp, wl.variant, half, wl.T)), wl.variant, 256, c0=st)
    got = np.concatenate([np.stack([h_f64(h[b, hh]) for b, hh in heads]) for h in (h1, h2)], axis=1)[None]
    err = rel_err(got, h_ref)
    print(f"rel err {err:.3e}", flush=True)
    assert err <= TOL[BF]
    got_c = np.stack([st[b, hh].cpu().double().numpy() for b, hh in heads])[None]
    assert rel_err(got_c, c_ref) <= STOL[BF]


# ---------------------------------------------------------------- segmented state walk
@pytest.mark.parametrize("segments", ["1", "2", "3", "7"])
@pytest.mark.parametrize("variant,dtype,B,H,T,dqk,dhv,L,with_c0", [
    (SIG, BF, 1, 2, 1500, 128, 128, 64, True),     # 24 chunks, partial last chunk
    (SIG, BF, 1, 1, 2048, 256, 512, 128, False),
    (SCAL, BF, 2, 1, 1000, 128, 256, 64, True),
    (GLA, BF, 1, 2, 900, 128, 128, 64, True),
    (SIG, F32, 1, 2, 1111, 64, 128, 64, True),
])
def test_segmented_state_walk(set_knob, segments, variant, dtype, B, H, T, dqk, dhv, L, with_c0):
    """The chunk chain cut into segments (end states from zero, a combine
    pass, a second walk from the true start states) gives the oracle's
    outputs, final state and chunk-boundary states."""
    set_knob(tfla.KNOB_STATE_SEGMENTS, segments)
    wl, inp = case(variant, B, H, T, dqk, dhv, dtype, seed=int(segments) * 100 + T)
    c0 = W.initial_state(B, H, dqk, dhv, seed=int(segments), std=1.5) if with_c0 else None
    print(f"segments {segments}: {variant} {dtype} B{B} H{H} T{T} {dqk}x{dhv} L{L} c0={with_c0}", flush=True)
    h, cf = run_state(to_dev(inp), variant, L, c0=c0)
    h_ref, c_ref = oracle_state(inp, variant, c0)
    assert rel_err(h_f64(h), h_ref) <= TOL[dtype]
    assert rel_err(cf.cpu().double().numpy(), c_ref) <= STOL[dtype]
    if not with_c0:
        _, st_ref = oracle.recurrent_fwd(W.as_f64(inp["q"]), W.as_f64(inp["k"]), W.as_f64(inp["v"]),
                                         W.as_f64(inp["igate_pre"]), W.as_f64(inp["fgate_pre"]), variant, L=L)
        nc = -(-T // L)
        st = torch.full((B, H, nc - 1, dhv, dqk), float("nan"), device="cuda", dtype=dtype)
        d = to_dev(inp)
        tfla.tfla_dbg_states(d["k"], d["v"], d["igate_pre"], d["fgate_pre"], st, B, H, T, dqk, dhv, L,
                             tfla.variant_of(GATE[variant], dtype))
        torch.cuda.synchronize()
        assert rel_err(st.cpu().double().numpy().swapaxes(-1, -2), st_ref[:, :, :nc - 1]) <= STOL[dtype]


# The combine pass takes 4-, 8- or 16-byte pieces per thread, as many as
# keep 512 or more workgroups (d_qk d_hv / (4 x 256) per head, times the
# heads): these shapes reach 8 and 16 bytes, and the per-channel gate with 4
# and 16 key channels per workgroup (d_hv = 128 and 64).
@pytest.mark.parametrize("variant,B,H,T,dqk,dhv,L,with_c0,segments", [
    (SIG, 1, 2, 1100, 256, 512, 64, True, "3"),     # 8-byte pieces
    (SIG, 1, 4, 1100, 256, 512, 64, False, "7"),    # 16-byte pieces
    (SCAL, 1, 4, 1100, 256, 512, 128, True, "3"),   # 16-byte pieces, the two-pass form
    (GLA, 2, 8, 700, 128, 128, 64, True, "3"),      # 8-byte pieces, 4 channels per workgroup
    (GLA, 4, 8, 700, 256, 64, 64, False, "5"),      # 16-byte pieces, 16 channels per workgroup
])
def test_segmented_walk_wide_combine(set_knob, variant, B, H, T, dqk, dhv, L, with_c0, segments):
    """The segmented walk at shapes whose combine pass takes wider pieces
    per thread: the oracle's outputs, final state and (without C_0) the
    chunk-boundary states."""
    set_knob(tfla.KNOB_STATE_SEGMENTS, segments)
    wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=int(segments) * 31 + dqk + H)
    c0 = W.initial_state(B, H, dqk, dhv, seed=3, std=1.5) if with_c0 else None
    print(f"wide combine: {variant} B{B} H{H} T{T} {dqk}x{dhv} L{L} c0={with_c0} P={segments}", flush=True)
    h, cf = run_state(to_dev(inp), variant, L, c0=c0)
    h_ref, c_ref = oracle_state(inp, variant, c0)
    assert rel_err(h_f64(h), h_ref) <= TOL[BF]
    assert rel_err(cf.cpu().double().numpy(), c_ref) <= STOL[BF]
    if not with_c0:
        _, st_ref = oracle.recurrent_fwd(W.as_f64(inp["q"]), W.as_f64(inp["k"]), W.as_f64(inp["v"]),
                                         W.as_f64(inp["igate_pre"]), W.as_f64(inp["fgate_pre"]), variant, L=L)
        nc = -(-T // L)
        st = torch.full((B, H, nc - 1, dhv, dqk), float("nan"), device="cuda", dtype=BF)
        d = to_dev(inp)
        tfla.tfla_dbg_states(d["k"], d["v"], d["igate_pre"], d["fgate_pre"], st, B, H, T, dqk, dhv, L,
                             tfla.variant_of(GATE[variant], BF))
        torch.cuda.synchronize()
        assert rel_err(st.cpu().double().numpy().swapaxes(-1, -2), st_ref[:, :, :nc - 1]) <= STOL[BF]


@pytest.mark.parametrize("variant,dtype,dqk,dhv,L,with_c0", [
    (SIG, BF, 128, 128, 64, True), (SCAL, BF, 128, 256, 64, False), (GLA, BF, 64, 128, 128, True),
    (SIG, F32, 64, 128, 64, True), (SIG, BF, 256, 512, 256, True),
])
@pytest.mark.parametrize("segments", ["2", "5"])
def test_segmented_walk_fixup_against_second_walk(set_knob, variant, dtype, dqk, dhv, L, with_c0, segments):
    """The forward segmented walk fixes up the states it stored (the start
    state of each segment, decayed, added in place); the two-pass form walks
    every segment again from its true start.  Both give the oracle's h and
    C_T, and the stored states of the two agree to within the one extra
    rounding of the fix-up (two roundings to the state type instead of one).
    The fixed decay walks twice either way."""
    set_knob(tfla.KNOB_STATE_SEGMENTS, segments)
    B, H, T = 1, 2, 64 * 23 + 17
    wl, inp = case(variant, B, H, T, dqk, dhv, dtype, seed=int(segments) * 7 + dqk + L)
    c0 = W.initial_state(B, H, dqk, dhv, seed=5, std=1.5) if with_c0 else None
    print(f"fix-up vs second walk: {variant} {dtype} {dqk}x{dhv} L{L} c0={with_c0} P={segments}", flush=True)
    h_ref, c_ref = oracle_state(inp, variant, c0)
    outs = {}
    for rewalk in (0, 1):
        with tfla.knob(tfla.KNOB_STATE_REWALK, rewalk):
            h, cf = run_state(to_dev(inp), variant, L, c0=c0)
            assert rel_err(h_f64(h), h_ref) <= TOL[dtype]
            assert rel_err(cf.cpu().double().numpy(), c_ref) <= STOL[dtype]
            if not with_c0:
                nc = -(-T // L)
                st = torch.full((B, H, nc - 1, dhv, dqk), float("nan"), device="cuda", dtype=dtype)
                d = to_dev(inp)
                tfla.tfla_dbg_states(d["k"], d["v"], d["igate_pre"], d["fgate_pre"], st, B, H, T, dqk, dhv, L,
                                     tfla.variant_of(GATE[variant], dtype))
                torch.cuda.synchronize()
                outs[rewalk] = st.double().cpu().numpy()
    if outs:
        unit = 2.0 ** -8 if dtype == BF else 2.0 ** -23   # the state type's relative spacing
        assert rel_err(outs[0], outs[1]) <= 2 * unit

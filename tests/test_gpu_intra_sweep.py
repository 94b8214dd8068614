"""The value-sweeping intra-chunk kernel (bf16 I/O, 64-, 128- or 256-step chunks,
two or more 128-wide value tiles: one workgroup per chunk forms P once and
sweeps every value tile) against the per-tile kernel it replaces there
(the intra-sweep test override selects that one), in the forward pass (every gate) and
in the backward pass's dv product.  Both take the same
products in the same order with the same roundings, so h (and every
gradient) must agree to the bit; both must match the oracle."""

import pytest
import torch

import workloads as W
from gpu_helpers import GATE, TOL, case, gpu_forward, h_f64, oracle_forward, rel_err, to_dev
from mlstm_sequence_amd import tfla

pytestmark = pytest.mark.gpu

SIG, SCAL, GLA = W.MLSTM_SIG, W.SCALAR, W.GLA
BF = torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tfla.lib()


def per_tile_kernel():
    """The per-tile kernel where the value sweep would run (test override)."""
    return tfla.knob(tfla.KNOB_INTRA_SWEEP, 0)


CASES = [
    # variant, B, H, T, dqk, dhv, L
    (SIG, 1, 2, 700, 256, 512, 256),    # ragged last chunk
    (SIG, 2, 1, 512, 256, 256, 256),    # two full chunks
    (SIG, 1, 2, 200, 256, 512, 256),    # one partial chunk: no inter-chunk term
    (SIG, 1, 1, 1, 256, 256, 256),      # a single step
    (SIG, 1, 2, 257, 128, 384, 256),    # one step into the second chunk; three value tiles
    (SIG, 1, 2, 900, 64, 256, 256),
    (SCAL, 2, 2, 600, 128, 256, 256),
    (SCAL, 1, 2, 1000, 256, 512, 256),
    (SIG, 1, 2, 300, 256, 512, 64),     # two-wave workgroups
    (SIG, 1, 1, 65, 128, 256, 64),
    (SCAL, 2, 1, 200, 256, 256, 64),
    (GLA, 1, 2, 300, 256, 512, 64),     # per-channel gate, the shape of its workload
    (GLA, 1, 1, 1, 256, 256, 64),
    (GLA, 2, 1, 130, 64, 384, 64),
    (GLA, 1, 2, 600, 128, 256, 256),    # per-channel gate at 8 waves (d_qk <= 128)
    (GLA, 1, 1, 300, 64, 512, 256),
    (SIG, 1, 2, 500, 256, 512, 128),    # four-wave workgroups
    (SCAL, 1, 2, 129, 128, 256, 128),
    (GLA, 1, 2, 400, 128, 256, 128),
]


@pytest.mark.parametrize("variant,B,H,T,dqk,dhv,L", CASES)
def test_sweep_matches_per_tile_kernel_and_oracle(variant, B, H, T, dqk, dhv, L):
    print(f"value sweep: variant {variant} B{B} H{H} T{T} {dqk}x{dhv} L{L}", flush=True)
    wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=7 * T + dqk + dhv)
    h_sweep = gpu_forward(inp, variant, L)
    with per_tile_kernel():
        h_tile = gpu_forward(inp, variant, L)
    assert torch.equal(h_sweep, h_tile)
    assert rel_err(h_f64(h_sweep), oracle_forward(inp, variant)) <= TOL[BF]


@pytest.mark.parametrize("variant,flags,L", [(SIG, 0, 256), (SCAL, 0, 256), (SIG, tfla.STATES_FP32, 256),
                                             (SIG, 0, 64), (GLA, 0, 64), (GLA, tfla.STATES_FP32, 64)])
def test_sweep_with_initial_state(variant, flags, L):
    B, H, T, dqk, dhv = 1, 2, 600, 256, 256
    print(f"value sweep with C_0: variant {variant} flags {flags:#x} L{L}", flush=True)
    wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=91)
    d = to_dev(inp)
    c0 = W.initial_state(B, H, dqk, dhv, seed=3, std=1.5).cuda()
    var = tfla.variant_of(GATE[variant], BF) | flags
    outs = []
    for sweep in (True, False):
        h = torch.full((B, H, T, dhv), float("nan"), dtype=BF, device="cuda")
        cf = torch.full((B, H, dqk, dhv), float("nan"), device="cuda")
        if sweep:
            tfla.tfla_fwd_state(d["q"], d["k"], d["v"], d["igate_pre"], d["fgate_pre"], c0, h, cf, B, H, T, dqk,
                                dhv, L, var)
        else:
            with per_tile_kernel():
                tfla.tfla_fwd_state(d["q"], d["k"], d["v"], d["igate_pre"], d["fgate_pre"], c0, h, cf, B, H, T,
                                    dqk, dhv, L, var)
        torch.cuda.synchronize()
        outs.append(h)
    assert torch.equal(outs[0], outs[1])
    assert bool(torch.isfinite(outs[0]).all())


@pytest.mark.parametrize("cfg,L", [(3, 256), (3, 128), (3, 64), (4, 64)])
def test_sweep_full_size(cfg, L):
    """Workload 3 (mLSTMsig B=4 H=8 T=8192 d_qk=256 d_hv=512; L = 256 is the
    launch the bench times) and workload 4 (per-channel gate B=8 H=4 T=2048
    d_qk=256 d_hv=512, L = 64) at full size."""
    wl = W.WORKLOADS[cfg]
    print(f"value sweep full size: {wl.name} L{L}", flush=True)
    inp = W.make_inputs(wl, device="cuda")
    h_sweep = gpu_forward(inp, wl.variant, L)
    with per_tile_kernel():
        h_tile = gpu_forward(inp, wl.variant, L)
    assert bool(torch.isfinite(h_sweep).all())
    assert torch.equal(h_sweep, h_tile)


# ---- the dv product of the backward pass (mirrored chunks) -----------------
from test_gpu_bwd import check as check_bwd, gpu_bwd, oracle_bwd          # noqa: E402
from test_gpu_bwd_state import gpu_bwd_state, states                       # noqa: E402


def same(a, b):
    for x, y in zip(a, b):
        assert (x is None) == (y is None)
        if x is not None:
            assert torch.equal(x, y)


@pytest.mark.parametrize("variant,B,H,T,dqk,dhv,L", [
    (SIG, 1, 2, 700, 256, 512, 256), (SCAL, 2, 1, 600, 128, 256, 256), (SIG, 1, 1, 200, 64, 256, 256),
    (SIG, 1, 2, 512, 256, 256, 256), (SIG, 1, 2, 300, 256, 512, 64), (SCAL, 1, 2, 150, 128, 256, 64),
    (GLA, 1, 2, 300, 256, 512, 64),     # per-channel gate (mirrored reference rows)
    (GLA, 2, 1, 333, 128, 256, 64), (GLA, 1, 2, 600, 128, 256, 256), (SIG, 1, 2, 500, 256, 512, 128),
    (GLA, 1, 1, 300, 128, 256, 128),
])
def test_dv_sweep_matches_per_tile_kernel_and_oracle(variant, B, H, T, dqk, dhv, L):
    print(f"dv value sweep: variant {variant} B{B} H{H} T{T} {dqk}x{dhv} L{L}", flush=True)
    wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=11 * T + dqk)
    dh = W.upstream_grad(B, H, T, dhv, BF, seed=T + 7)
    got = gpu_bwd(inp, dh, variant, L, workspace=True)
    with per_tile_kernel():
        ref_tile = gpu_bwd(inp, dh, variant, L, workspace=True)
    same(got, ref_tile)
    check_bwd(got, oracle_bwd(inp, dh, variant), BF, "sweep")


@pytest.mark.parametrize("variant,L", [(SIG, 256), (SCAL, 256), (SIG, 64), (GLA, 64)])
def test_dv_sweep_with_initial_state_and_final_state_gradient(variant, L):
    B, H, T, dqk, dhv = 1, 2, 600, 256, 256
    print(f"dv value sweep with C_0 and dL/dC_T: variant {variant} L{L}", flush=True)
    wl, inp = case(variant, B, H, T, dqk, dhv, BF, seed=123)
    dh = W.upstream_grad(B, H, T, dhv, BF, seed=9)
    c0, g = states(B, H, dqk, dhv, 77, True, True)
    got = gpu_bwd_state(inp, dh, variant, L, c0=c0, dcT=g)
    with per_tile_kernel():
        ref_tile = gpu_bwd_state(inp, dh, variant, L, c0=c0, dcT=g)
    same(got, ref_tile)


def test_sweep_more_than_2_31_elements():
    """v and h hold 64 * 65536 * 512 = 2^31 elements; the last head sits past
    every 32-bit offset (inputs drawn on the GPU by the seeded generators)."""
    import numpy as np
    B, H, T = 1, 64, 65536
    wl = W.WORKLOADS[5].with_(B=B, H=H, T=T, dqk=256, dhv=512, seed=53)
    print(f"value sweep, 2^31 elements: B{B} H{H} T{T} 256x512 L256", flush=True)
    inp = W.make_inputs(wl, device="cuda")
    assert inp["v"].numel() == 1 << 31
    h = gpu_forward(inp, wl.variant, 256, workspace=True)
    assert bool(torch.isfinite(h).all())
    heads = [(0, H - 1)]
    sl = {k: (None if t is None else t.cpu()) for k, t in W.head_slice(inp, wl.variant, heads).items()}
    del inp
    ref = oracle_forward(sl, wl.variant)
    got = np.stack([h_f64(h[b, hh]) for b, hh in heads])
    err = rel_err(got, ref)
    print(f"rel err {err:.3e}", flush=True)
    assert err <= TOL[BF]

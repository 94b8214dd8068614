"""mLSTMexp (exponential input gate, normaliser state, max state; forward
only) on the GPU against its CPU oracle (oracle_fwd_exp), element by element
over the whole output: both intra-chunk kernels (the value sweep and the
per-tile kernel), fp32 and bf16 I/O, ragged sequences, input gates that keep
the normaliser below 1 and ones that drive it far above, fp32 states, the
segmented state walk, and the T = 8192 head shape at full size."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, h_f64, rel_err, to_dev
from mlstm_sequence_amd import tfla

pytestmark = pytest.mark.gpu

BF, F32 = torch.bfloat16, torch.float32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tfla.lib()


def exp_case(B, H, T, dqk, dhv, dtype, seed, ig_mean=0.0):
    """mLSTMsig inputs of the T = 8192 workload's distributions (q, k, v ~
    N(0,1), igate_pre ~ N(ig_mean, 1), fgate_pre ~ U(3, 6)), read as mLSTMexp
    pre-activations."""
    wl = W.WORKLOADS[3].with_(B=B, H=H, T=T, dqk=dqk, dhv=dhv, dtype=dtype, seed=seed, igate_mean=ig_mean)
    return wl, W.make_inputs(wl)


def run_exp(inp, L, flags=0, workspace=False):
    d = to_dev(inp)
    q, v = d["q"], d["v"]
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    var = tfla.variant_of(tfla.MLSTM_EXP, q.dtype) | flags
    h = torch.full((B, H, T, dhv), float("nan"), dtype=q.dtype, device="cuda")
    if workspace:
        n = tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, L, var)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
        tfla.tfla_fwd_ws(q, d["k"], v, d["igate_pre"], d["fgate_pre"], h, B, H, T, dqk, dhv, L, var, ws, n)
    else:
        tfla.tfla_fwd(q, d["k"], v, d["igate_pre"], d["fgate_pre"], h, B, H, T, dqk, dhv, L, var)
    torch.cuda.synchronize()
    return h


def oracle_exp(inp):
    return oracle.recurrent_fwd_exp(W.as_f64(inp["q"]), W.as_f64(inp["k"]), W.as_f64(inp["v"]),
                                    W.as_f64(inp["igate_pre"]), W.as_f64(inp["fgate_pre"]))


CASES = [
    # dtype, B, H, T, dqk, dhv, L, igate mean
    (BF, 1, 2, 600, 256, 512, 256, 0.0),     # value sweep, 8 waves: the T = 8192 workload's launch
    (BF, 1, 2, 300, 128, 256, 128, 0.0),     # value sweep, 4 waves
    (BF, 2, 1, 200, 64, 256, 64, 0.0),       # value sweep, 2 waves
    (BF, 1, 2, 333, 128, 128, 64, 0.0),      # per-tile kernel (one value tile)
    (BF, 1, 2, 1100, 256, 512, 512, 0.0),    # per-tile kernel, long chunks
    (BF, 1, 1, 2100, 128, 256, 1024, 0.0),
    (BF, 1, 2, 1, 128, 256, 64, 0.0),        # one step
    (BF, 1, 2, 65, 256, 512, 256, 0.0),      # a partial first chunk only
    (BF, 1, 2, 700, 256, 512, 256, -10.0),   # input-gate bias -10: the normaliser stays below 1
    (BF, 1, 2, 700, 256, 512, 256, 20.0),    # strong input gates: e^20 and more, max state at work
    (BF, 1, 2, 500, 128, 192, 128, 5.0),
    (F32, 1, 1, 256, 64, 64, 64, 0.0),       # fp32 I/O
    (F32, 1, 2, 300, 128, 256, 128, 3.0),
    (F32, 2, 1, 1025, 64, 128, 512, -4.0),
]


@pytest.mark.parametrize("dtype,B,H,T,dqk,dhv,L,ig", CASES)
def test_exp_matches_oracle(dtype, B, H, T, dqk, dhv, L, ig):
    print(f"mLSTMexp {dtype} B{B} H{H} T{T} {dqk}x{dhv} L{L} igate mean {ig}", flush=True)
    wl, inp = exp_case(B, H, T, dqk, dhv, dtype, seed=T + dqk + int(ig), ig_mean=ig)
    h = run_exp(inp, L, workspace=(T % 2 == 0))
    assert bool(torch.isfinite(h).all())
    err = rel_err(h_f64(h), oracle_exp(inp))
    print(f"  rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]


def test_exp_fp32_states_give_the_same_h():
    wl, inp = exp_case(1, 2, 700, 256, 512, BF, seed=5)
    h16 = run_exp(inp, 256)
    h32 = run_exp(inp, 256, flags=tfla.STATES_FP32)
    assert torch.equal(h16, h32)


@pytest.mark.parametrize("segments", [2, 5])
def test_exp_segmented_state_walk(segments, set_knob):
    """Few heads, many chunks: the state walk cut into segments (end states
    from zero, a combine pass, a second walk) over mLSTMexp's exponents."""
    set_knob(tfla.KNOB_STATE_SEGMENTS, segments)
    wl, inp = exp_case(1, 2, 64 * 11 + 29, 64, 128, BF, seed=segments)
    print(f"mLSTMexp segments {segments}", flush=True)
    h = run_exp(inp, 64)
    assert rel_err(h_f64(h), oracle_exp(inp)) <= TOL[BF]


def test_exp_full_size_sampled_heads():
    """B=4 H=8 T=8192 d_qk=256 d_hv=512 bf16 at L = 256 (the T = 8192
    workload's shape and launch), sampled heads against the oracle."""
    wl = W.WORKLOADS[3]
    inp = W.make_inputs(wl)
    heads = [(0, 0), (3, 7)]
    print("mLSTMexp full size", flush=True)
    h = run_exp(inp, 256, workspace=True)
    assert bool(torch.isfinite(h).all())
    sl = W.head_slice(inp, wl.variant, heads)
    ref = oracle_exp(sl)
    got = np.stack([h_f64(h[b, hh]) for b, hh in heads])[None]
    err = rel_err(got, ref)
    print(f"  rel err {err:.3e}", flush=True)
    assert err <= TOL[BF]

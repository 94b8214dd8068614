"""Parity at the size limits of the API: the largest head count (B*H = 65535)
for the forward and the backward pass, and tensors of more than 2^31
elements (every index past 32 bits).  The inputs are drawn on the GPU by the
seeded generators of workloads.py (too large to draw on the host); the oracle
recomputes sampled heads, the first and the last among them, element by
element; every other head must be written (NaN prefill) and finite."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, gpu_forward, h_f64, oracle_forward, rel_err
from test_gpu_bwd import gpu_bwd

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def sampled(inp, variant, heads):
    return {k: (None if t is None else t.cpu()) for k, t in W.head_slice(inp, variant, heads).items()}


@pytest.mark.parametrize("variant", [W.MLSTM_SIG, W.GLA])
def test_largest_head_count_forward(variant):
    B, H, T = 5, 13107, 130                     # B*H = 65535, a ragged third chunk at L = 64
    wl = W.WORKLOADS[3 if variant == W.MLSTM_SIG else 4].with_(B=B, H=H, T=T, dqk=64, dhv=64, seed=41)
    print(f"largest head count: variant {variant} B{B} H{H} T{T} 64x64 L64", flush=True)
    inp = W.make_inputs(wl, device="cuda")
    h = gpu_forward(inp, variant, 64)
    assert bool(torch.isfinite(h).all())
    heads = [(0, 0), (2, 6553), (B - 1, H - 1)]
    ref = oracle_forward(sampled(inp, variant, heads), variant)[0]
    got = np.stack([h_f64(h[b, hh]) for b, hh in heads])
    err = rel_err(got, ref)
    print(f"rel err {err:.3e}", flush=True)
    assert err <= TOL[BF]


def test_largest_head_count_backward():
    B, H, T = 5, 13107, 130
    wl = W.WORKLOADS[3].with_(B=B, H=H, T=T, dqk=64, dhv=64, seed=43)
    print(f"largest head count, backward: B{B} H{H} T{T} 64x64 L64", flush=True)
    inp = W.make_inputs(wl, device="cuda")
    dh = W.upstream_grad(B, H, T, 64, BF, seed=44, device="cuda")
    got = gpu_bwd(inp, dh, W.MLSTM_SIG, 64, workspace=True)
    for g in got:
        assert bool(torch.isfinite(g).all())
    heads = [(0, 0), (B - 1, H - 1)]
    sl = sampled(inp, W.MLSTM_SIG, heads)
    dh_sl = torch.stack([dh[b, hh] for b, hh in heads])[None].cpu()
    ref = oracle.recurrent_bwd(W.as_f64(sl["q"]), W.as_f64(sl["k"]), W.as_f64(sl["v"]), W.as_f64(sl["igate_pre"]),
                               W.as_f64(sl["fgate_pre"]), W.as_f64(dh_sl), W.MLSTM_SIG)
    for name, g, r in zip(["dq", "dk", "dv", "dig", "dfg"], got, ref):
        mine = np.stack([h_f64(g[b, hh]) for b, hh in heads])[None]
        err = rel_err(mine, r)
        print(f"  {name}: {err:.3e}", flush=True)
        assert err <= TOL[BF], name


def test_more_than_2_31_elements_forward():
    # v and h hold 512 * 65536 * 64 = 2^31 elements each; the last head's
    # elements sit past every 32-bit offset
    B, H, T = 1, 512, 65536
    wl = W.WORKLOADS[5].with_(B=B, H=H, T=T, dqk=64, dhv=64, seed=47)
    print(f"2^31 elements: B{B} H{H} T{T} 64x64 L256", flush=True)
    inp = W.make_inputs(wl, device="cuda")
    assert inp["v"].numel() == 1 << 31
    h = gpu_forward(inp, W.MLSTM_SIG, 256, workspace=True)
    assert bool(torch.isfinite(h).all())
    heads = [(0, 0), (0, H - 1)]
    ref = oracle_forward(sampled(inp, W.MLSTM_SIG, heads), W.MLSTM_SIG)[0]
    got = np.stack([h_f64(h[b, hh]) for b, hh in heads])
    err = rel_err(got, ref)
    print(f"rel err {err:.3e}", flush=True)
    assert err <= TOL[BF]

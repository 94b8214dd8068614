"""Backward parity at the full workload sizes with a caller-owned workspace:
the GPU runs the whole workload, the oracle's backward recurrence recomputes
a sample of heads over their whole sequences, and those heads are compared
element by element (tolerances of the forward pass).  The per-head
scalar-decay gradient sums over batches, so its sample takes every batch of
the sampled heads."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, h_f64, rel_err
from test_gpu_bwd import gpu_bwd

pytestmark = pytest.mark.gpu

# (workload, chunk size, sampled (b, h) heads); the T = 8192 mLSTMsig
# workload also at the longest chunk its benchmark sweep reports
CASES = [
    (1, 64, [(0, 0)]),
    (2, 64, [(b, 17) for b in range(8)]),
    (3, 256, [(0, 0), (3, 7)]),
    (3, 1024, [(1, 2)]),
    (4, 64, [(0, 0), (7, 3)]),
    (5, 256, [(0, 5)]),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("c,L,heads", CASES, ids=[f"cfg{c}-L{L}" for c, L, _ in CASES])
def test_full_size_backward_sampled_heads(c, L, heads):
    wl = W.WORKLOADS[c]
    inp = W.make_inputs(wl)
    dh = W.upstream_grad(wl.B, wl.H, wl.T, wl.dhv, wl.dtype, seed=wl.seed + 1)
    print(f"backward {wl.name} L={L} heads {heads}", flush=True)
    got = gpu_bwd(inp, dh, wl.variant, L, workspace=True)
    for g in got:
        if g is not None:
            assert bool(torch.isfinite(g).all())
    sl = W.head_slice(inp, wl.variant, heads)
    dh_sl = torch.stack([dh[b, h] for b, h in heads])[None]
    print("oracle ...", flush=True)
    ref = oracle.recurrent_bwd(W.as_f64(sl["q"]), W.as_f64(sl["k"]), W.as_f64(sl["v"]), W.as_f64(sl["igate_pre"]),
                               W.as_f64(sl["fgate_pre"]), W.as_f64(dh_sl), wl.variant)
    for name, g, r in zip(["dq", "dk", "dv", "dig"], got[:4], ref[:4]):
        if r is None:
            continue
        mine = np.stack([h_f64(g[b, h]) for b, h in heads])[None]
        err = rel_err(mine, r)
        print(f"  {name}: {err:.3e}", flush=True)
        assert err <= TOL[wl.dtype], name
    if wl.variant == W.SCALAR:
        # dfg[h] of the library sums every batch; the slice's per-head entries sum to it
        h = heads[0][1]
        err = rel_err(h_f64(got[4])[h], np.sum(ref[4]))
    else:
        mine = np.stack([h_f64(got[4][b, h]) for b, h in heads])[None]
        err = rel_err(mine, ref[4])
    print(f"  dfg: {err:.3e}", flush=True)
    assert err <= TOL[wl.dtype]

"""Parity at the full workload sizes, in the launch configuration the
benchmark times (caller-owned workspace, tfla_fwd_ws).  The GPU runs the
whole workload; the oracle recomputes a sample of heads, each over its whole
sequence, and those heads are compared element by element.  Every other
head is checked for finiteness and for having been written (NaN prefill)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import TOL, gpu_forward, h_f64, oracle_forward, rel_err

pytestmark = pytest.mark.gpu

SAMPLES = {1: [(0, 0)], 2: [(0, 0), (3, 17), (7, 31)], 3: [(0, 0), (3, 7)], 4: [(0, 0), (7, 3)],
           5: [(0, 0), (0, 7)]}
# every listed chunk size, plus the longer chunks the benchmark's sweep
# reports for the T = 8192 mLSTMsig workload (d_qk = 256, d_hv = 512)
CASES = sorted([(c, L) for c in W.WORKLOADS for L in W.WORKLOADS[c].chunk_sizes] + [(3, 512), (3, 1024)])

_cache = {}


def inputs_and_reference(c):
    if c not in _cache:
        _cache.clear()                       # keep one workload's inputs in memory
        wl = W.WORKLOADS[c]
        inp = W.make_inputs(wl)
        heads = SAMPLES[c]
        ref = oracle_forward(W.head_slice(inp, wl.variant, heads), wl.variant)[0]
        _cache[c] = (wl, inp, heads, ref)
    return _cache[c]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("c,L", CASES, ids=[f"cfg{c}-L{L}" for c, L in CASES])
def test_full_size_sampled_heads(c, L):
    wl, inp, heads, ref = inputs_and_reference(c)
    print(f"workload {wl.name} L={L} heads {heads}", flush=True)
    h = gpu_forward(inp, wl.variant, L, workspace=True)
    assert bool(torch.isfinite(h).all())
    got = np.stack([h_f64(h[b, hh]) for b, hh in heads])
    err = rel_err(got, ref)
    print(f"rel err {err:.3e}", flush=True)
    assert err <= TOL[wl.dtype]

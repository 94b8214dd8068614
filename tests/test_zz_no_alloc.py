"""tfla_fwd_noalloc: the forward pass with the library's static scratch as its
workspace (for callers that cannot allocate).  Two calls in a row, the second
with a smaller problem, each against tfla_fwd (the allocating entry point) on
the same inputs -- bitwise, since both run the same kernels on the same
workspace layout -- and against the oracle at the forward pass's tolerance."""
import pytest
import torch

from gpu_helpers import GATE, TOL, case, h_f64, oracle_forward, rel_err, to_dev
from mlstm_sequence_amd import tfla
from workloads import GLA, MLSTM_SIG, SCALAR

pytestmark = pytest.mark.gpu

BF, F32 = torch.bfloat16, torch.float32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tfla.lib()


def run(entry, d, variant, L):
    q, v = d["q"], d["v"]
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    h = torch.full((B, H, T, dhv), float("nan"), dtype=q.dtype, device="cuda")
    entry(q, d["k"], v, d["igate_pre"], d["fgate_pre"], h, B, H, T, dqk, dhv, L,
          tfla.variant_of(GATE[variant], q.dtype))
    return h


# (first call, second call): the second problem is smaller than the first
PAIRS = [
    ((MLSTM_SIG, BF, 2, 3, 1100, 128, 256, 256), (MLSTM_SIG, BF, 1, 2, 300, 64, 128, 64)),
    ((GLA, BF, 1, 4, 900, 128, 256, 64), (SCALAR, BF, 1, 2, 200, 128, 128, 128)),
    ((MLSTM_SIG, F32, 1, 2, 64 * 20 + 7, 64, 128, 64), (MLSTM_SIG, F32, 1, 1, 256, 64, 64, 64)),
]


@pytest.mark.parametrize("first,second", PAIRS, ids=["sig", "gla-then-scalar", "fp32-segmented"])
def test_noalloc_matches_the_allocating_entry_point(first, second):
    assert tfla.tfla_fwd_noalloc_max_workspace() == 64 << 20
    for variant, dtype, B, H, T, dqk, dhv, L in (first, second):
        wl, inp = case(variant, B, H, T, dqk, dhv, dtype, seed=T + dqk)
        d = to_dev(inp)
        need = tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, L, tfla.variant_of(GATE[variant], dtype))
        print(f"noalloc {variant} {dtype} B{B} H{H} T{T} {dqk}x{dhv} L{L} workspace {need} B", flush=True)
        h_na = run(tfla.tfla_fwd_noalloc, d, variant, L)
        torch.cuda.synchronize()
        h_ref = run(tfla.tfla_fwd, d, variant, L)
        torch.cuda.synchronize()
        assert torch.equal(h_na, h_ref)
        err = rel_err(h_f64(h_na), oracle_forward(inp, variant))
        print(f"  rel err {err:.3e}", flush=True)
        assert err <= TOL[dtype]


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    B, H, T, dqk, dhv, L = 4, 8, 8192, 256, 512, 64          # ~1 GB of states
    var = tfla.variant_of(tfla.MLSTM_SIG, BF)
    assert tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, L, var) > tfla.tfla_fwd_noalloc_max_workspace()
    q = torch.empty((B, H, T, dqk), dtype=BF, device="cuda")
    v = torch.empty((B, H, T, dhv), dtype=BF, device="cuda")
    g = torch.zeros((B, H, T), device="cuda")
    h = torch.empty_like(v)
    with pytest.raises(tfla.TflaError) as e:
        tfla.tfla_fwd_noalloc(q, q, v, g, g, h, B, H, T, dqk, dhv, L, var)
    assert e.value.code == tfla.ERR_OUT_OF_MEMORY and "scratch" in str(e.value)

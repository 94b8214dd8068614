"""fp32 I/O at the widest head dimensions (d_qk = 256, d_hv up to 512), forward
and backward, against the oracle at the fp32 bar (1e-4): the per-tile intra
kernel with 64-wide value tiles, the 64 x 64 state tiles, and in the backward
pass the shared P, which the 256- and 512-wide fp32 contractions of dq and dk
take so that their Q fragments need not be held."""
import pytest
import torch

from gpu_helpers import TOL, case, gpu_forward, h_f64, oracle_forward, rel_err
from mlstm_sequence_amd import tfla
from workloads import GLA, MLSTM_SIG, SCALAR

pytestmark = pytest.mark.gpu

F32 = torch.float32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tfla.lib()


FWD = [
    # variant, B, H, T, dqk, dhv, L
    (MLSTM_SIG, 1, 2, 300, 256, 512, 64),
    (MLSTM_SIG, 1, 1, 700, 256, 512, 256),
    (MLSTM_SIG, 1, 1, 1100, 256, 320, 512),
    (SCALAR, 1, 2, 260, 256, 384, 128),
    (GLA, 1, 1, 200, 256, 512, 64),
    (MLSTM_SIG, 1, 2, 333, 128, 512, 128),
]


@pytest.mark.parametrize("variant,B,H,T,dqk,dhv,L", FWD)
def test_fp32_wide_forward(variant, B, H, T, dqk, dhv, L):
    print(f"fp32 wide forward: variant {variant} B{B} H{H} T{T} {dqk}x{dhv} L{L}", flush=True)
    wl, inp = case(variant, B, H, T, dqk, dhv, F32, seed=T + dqk + dhv)
    h = gpu_forward(inp, variant, L, workspace=True)
    err = rel_err(h_f64(h), oracle_forward(inp, variant))
    print(f"  rel err {err:.3e}", flush=True)
    assert err <= TOL[F32]


BWD = [
    (MLSTM_SIG, 1, 2, 200, 256, 256, 64),
    (MLSTM_SIG, 1, 1, 300, 128, 512, 128),
    (MLSTM_SIG, 1, 1, 260, 64, 512, 64),      # one value tile of d_qk: P is shared anyway
    (SCALAR, 1, 2, 150, 256, 512, 64),
    (GLA, 1, 1, 130, 256, 256, 64),
    (GLA, 1, 1, 100, 64, 512, 64),            # the per-channel gate never shares P: fp32 Q fragments spill
]


@pytest.mark.parametrize("variant,B,H,T,dqk,dhv,L", BWD)
def test_fp32_wide_backward(variant, B, H, T, dqk, dhv, L):
    from test_gpu_bwd import check, gpu_bwd, oracle_bwd
    import workloads as W
    print(f"fp32 wide backward: variant {variant} B{B} H{H} T{T} {dqk}x{dhv} L{L}", flush=True)
    wl, inp = case(variant, B, H, T, dqk, dhv, F32, seed=3 * T + dqk + dhv)
    dh = W.upstream_grad(B, H, T, dhv, F32, seed=T + 2)
    got = gpu_bwd(inp, dh, variant, L, workspace=True)
    check(got, oracle_bwd(inp, dh, variant), F32, "bwd")

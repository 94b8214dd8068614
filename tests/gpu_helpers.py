"""Shared helpers of the GPU tests: run the library on seeded inputs and
compare with the CPU oracle."""
import math

import numpy as np
import torch

import oracle
import workloads as W
from mlstm_sequence_amd import tfla

GATE = {W.MLSTM_SIG: tfla.MLSTM_SIG, W.SCALAR: tfla.SCALAR_DECAY, W.GLA: tfla.GLA_KEY}
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    d = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    if not math.isfinite(d):
        return math.inf
    return d / (m if m > 0 else 1.0)


def to_dev(inp: dict) -> dict:
    return {k: (None if t is None else t.cuda()) for k, t in inp.items()}


def gpu_forward(inp: dict, variant: int, L: int, workspace: bool = False):
    """Runs the library; h is prefilled with NaN so every element must be written."""
    d = to_dev(inp)
    q, v = d["q"], d["v"]
    h = torch.full((q.shape[0], q.shape[1], q.shape[2], v.shape[-1]), float("nan"), dtype=q.dtype,
                   device=q.device)
    ws = tfla.workspace_for(q, v, GATE[variant], L) if workspace else None
    tfla.forward(q, d["k"], v, d["igate_pre"], d["fgate_pre"], GATE[variant], L, h=h, workspace=ws)
    torch.cuda.synchronize()
    return h


def oracle_forward(inp: dict, variant: int, L=None):
    return oracle.recurrent_fwd(W.as_f64(inp["q"]), W.as_f64(inp["k"]), W.as_f64(inp["v"]),
                                W.as_f64(inp["igate_pre"]), W.as_f64(inp["fgate_pre"]), variant, L=L)


def h_f64(h: torch.Tensor) -> np.ndarray:
    return h.detach().float().cpu().double().numpy()


def case(variant, B, H, T, dqk, dhv, dtype, seed, **kw) -> tuple:
    base = {W.MLSTM_SIG: W.WORKLOADS[3], W.SCALAR: W.WORKLOADS[2], W.GLA: W.WORKLOADS[4]}[variant]
    wl = base.with_(B=B, H=H, T=T, dqk=dqk, dhv=dhv, dtype=dtype, seed=seed, **kw)
    return wl, W.make_inputs(wl)

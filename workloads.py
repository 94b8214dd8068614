"""Seeded synthetic inputs shaped like the workloads on the pages.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no arithmetic of the method: it only draws random numbers with a seeded
CPU ``torch.Generator`` and casts them (fp32 draws, cast round-to-nearest-even
to bf16 for the bf16 workloads).  Both the GPU library and the CPU oracle
receive the very same values.  Inputs too large to draw on the host (the
size-limit tests) are drawn the same way by a seeded generator on the GPU;
the oracle then receives copies of the sampled heads.

Draw order for every workload: q, k, v, then the input-gate pre-activation
(mLSTMsig and mLSTMexp), then the forget-gate pre-activation (per step, or per step
and key channel for the per-channel gate).  The per-head scalar decay needs no
draw: gamma_h = 1 - 2^-(5 + h/4) (the decay schedule of the RetNet-style
multi-scale retention the flash-linear-attention README benchmarks), passed as
its logit ln(2^(5 + h/4) - 1), evaluated in float64 and rounded to fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

MLSTM_SIG, SCALAR, GLA, MLSTM_EXP = 0, 1, 2, 3
VARIANT_NAMES = {MLSTM_SIG: "mlstm_sig", SCALAR: "scalar_decay", GLA: "gla_key", MLSTM_EXP: "mlstm_exp"}


@dataclass(frozen=True)
class Workload:
    name: str
    variant: int
    B: int
    H: int
    T: int
    dqk: int
    dhv: int
    dtype: torch.dtype
    chunk_sizes: tuple
    qkv_std: float = 1.0
    igate_mean: float = 0.0
    fgate_range: tuple = (3.0, 6.0)      # uniform forget-gate pre-activation (mLSTMsig)
    seed: int = 0
    notes: str = field(default="", compare=False)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def dtype_name(self) -> str:
        return "bf16" if self.dtype == torch.bfloat16 else "fp32"


# The five workloads.  Seeds are 1000 + index.
WORKLOADS = {
    1: Workload("mlstm_sig_fp32_T256", MLSTM_SIG, 1, 1, 256, 64, 64, torch.float32, (64,),
                seed=1001, notes="tiny fp32 case"),
    2: Workload("scalar_decay_bf16_T4096", SCALAR, 8, 32, 4096, 128, 128, torch.bfloat16, (64,),
                qkv_std=1.0 / math.sqrt(128), seed=1002,
                notes="shape of the A100 RetNet timing table of the flash-linear-attention README"),
    3: Workload("mlstm_sig_bf16_T8192", MLSTM_SIG, 4, 8, 8192, 256, 512, torch.bfloat16,
                (64, 128, 256), seed=1003, notes="headline throughput workload"),
    4: Workload("gla_key_bf16_T2048", GLA, 8, 4, 2048, 256, 512, torch.bfloat16, (64,),
                qkv_std=1.0 / math.sqrt(256), seed=1004, notes="per-key-channel gate"),
    5: Workload("mlstm_sig_bf16_T65536", MLSTM_SIG, 1, 8, 65536, 128, 128, torch.bfloat16,
                (64, 128, 256, 512), igate_mean=-10.0, seed=1005,
                notes="long context, input-gate bias -10"),
}


def scalar_decay_logits(H: int) -> torch.Tensor:
    """fp32 logits of gamma_h = 1 - 2^-(5 + h/4), h = 0..H-1."""
    vals = [math.log(2.0 ** (5.0 + h / 4.0) - 1.0) for h in range(H)]
    return torch.tensor(vals, dtype=torch.float64).to(torch.float32)


def make_inputs(w: Workload, seed: int | None = None, device="cpu") -> dict:
    """Draws the inputs of ``w`` on ``device`` (the CPU unless a test asks for the GPU).  Returns a dict with q, k, v
    (``w.dtype``), igate_pre (fp32 [B,H,T] or None), fgate_pre (fp32)."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed if seed is None else seed)
    B, H, T = w.B, w.H, w.T

    def normal(shape, std=1.0, mean=0.0):
        x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
        if std != 1.0:
            x = x * torch.tensor(std, dtype=torch.float32)
        if mean != 0.0:
            x = x + torch.tensor(mean, dtype=torch.float32)
        return x

    q = normal((B, H, T, w.dqk), w.qkv_std).to(w.dtype)
    k = normal((B, H, T, w.dqk), w.qkv_std).to(w.dtype)
    v = normal((B, H, T, w.dhv), w.qkv_std).to(w.dtype)
    if w.variant in (MLSTM_SIG, MLSTM_EXP):
        ig = normal((B, H, T), 1.0, w.igate_mean)
        lo, hi = w.fgate_range
        fg = torch.rand((B, H, T), generator=g, dtype=torch.float32, device=device) * (hi - lo) + lo
    elif w.variant == SCALAR:
        ig = None
        fg = scalar_decay_logits(H).to(device)
    elif w.variant == GLA:
        ig = None
        fg = normal((B, H, T, w.dqk))
    else:
        raise ValueError(w.variant)
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "igate_pre": None if ig is None else ig.contiguous(), "fgate_pre": fg.contiguous()}


def as_f64(t) -> np.ndarray | None:
    """Exact float64 copy of a CPU tensor (bf16 and fp32 values are exact in
    float64)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def initial_state(B: int, H: int, dqk: int, dhv: int, seed: int, std: float = 1.0) -> torch.Tensor:
    """A seeded fp32 initial state C_0 [B,H,d_qk,d_hv] ~ N(0, std^2)."""
    g = torch.Generator().manual_seed(seed)
    return torch.randn((B, H, dqk, dhv), generator=g, dtype=torch.float32) * std


def upstream_grad(B: int, H: int, T: int, dhv: int, dtype: torch.dtype, seed: int, device="cpu") -> torch.Tensor:
    """A seeded gradient dL/dh [B,H,T,d_hv] ~ N(0, 1), cast to ``dtype``
    (the input of the backward pass)."""
    g = torch.Generator(device=device).manual_seed(seed)
    return torch.randn((B, H, T, dhv), generator=g, dtype=torch.float32, device=device).to(dtype).contiguous()


def head_slice(inputs: dict, variant: int, heads: list) -> dict:
    """Inputs restricted to a list of (b, h) pairs, as a batch of one with
    len(heads) heads -- used to run the oracle on sampled heads of a large
    workload.  The scalar-decay logits follow their heads."""
    def pick(t):
        return torch.stack([t[b, h] for b, h in heads])[None]

    out = {"q": pick(inputs["q"]), "k": pick(inputs["k"]), "v": pick(inputs["v"])}
    out["igate_pre"] = None if inputs["igate_pre"] is None else pick(inputs["igate_pre"])
    if variant == SCALAR:
        out["fgate_pre"] = torch.stack([inputs["fgate_pre"][h] for _, h in heads])
    else:
        out["fgate_pre"] = pick(inputs["fgate_pre"])
    return out

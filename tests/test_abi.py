"""The C-ABI boundary without a GPU: the library loads, exports every entry
point include/tfla.h declares, and rejects bad arguments before any HIP call
(so these run on a machine with no GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tfla.h")

tfla = pytest.importorskip("mlstm_sequence_amd.tfla")

BF16 = 0x100
SIG, SCALAR, GLA, EXP = 0, 1, 2, 3
INVALID, UNSUPPORTED, OOM = 1, 2, 4

# 16-byte aligned fake device addresses: validation never dereferences them
Q, K, V, H_, IG, FG, WS, C0, CF = (0x10000000 * (n + 1) for n in range(9))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tfla_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tfla.LIB_PATH):
        pytest.skip("libtfla.so not built")
    return tfla.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"tfla_fwd", "tfla_fwd_ws", "tfla_workspace_bytes", "tfla_dbg_gates", "tfla_dbg_states",
            "tfla_fwd_state", "tfla_state_workspace_bytes", "tfla_fwd_recurrent",
            "tfla_bwd", "tfla_bwd_workspace_bytes",
            "tfla_error_string", "tfla_last_error", "tfla_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings(L):
    assert tfla.tfla_version() == 300
    for code in range(5):
        assert tfla.error_string(code)
    assert tfla.error_string(99) == "unknown status code"


def fwd(q=Q, k=K, v=V, ig=IG, fg=FG, h=H_, B=2, H=3, T=300, dqk=128, dhv=256, Lc=64, variant=SIG | BF16):
    return tfla.lib().tfla_fwd(q, k, v, ig, fg, h, B, H, T, dqk, dhv, Lc, variant, None)


@pytest.mark.parametrize("kw,code", [
    (dict(variant=4), INVALID), (dict(variant=0x200), INVALID), (dict(variant=-1), INVALID),
    (dict(B=0), INVALID), (dict(T=0), INVALID), (dict(H=-2), INVALID),
    (dict(q=None), INVALID), (dict(h=None), INVALID), (dict(fg=None), INVALID),
    (dict(q=Q + 8), INVALID), (dict(h=H_ + 2), INVALID), (dict(fg=FG + 2), INVALID),
    (dict(variant=GLA | BF16, ig=None, fg=FG + 4), INVALID),   # per-channel gate rows: 16-byte aligned
    (dict(ig=None), INVALID),                                   # mLSTMsig needs an input gate
    (dict(ig=None, variant=EXP | BF16), INVALID),               # ... and so does mLSTMexp
    (dict(variant=SCALAR | BF16), INVALID),                     # ... the others must not have one
    (dict(h=Q + 64), INVALID), (dict(h=V - 32), INVALID),       # output overlaps an input
    (dict(dqk=96), UNSUPPORTED), (dict(dqk=512), UNSUPPORTED), (dict(dhv=100), UNSUPPORTED),
    (dict(dhv=576), UNSUPPORTED), (dict(Lc=32), UNSUPPORTED), (dict(Lc=96), UNSUPPORTED),
    (dict(Lc=2048), UNSUPPORTED), (dict(variant=SIG, dqk=512), UNSUPPORTED),
    (dict(variant=SIG, dhv=576), UNSUPPORTED), (dict(B=300, H=300), UNSUPPORTED),
])
def test_rejects_bad_arguments(L, kw, code):
    assert fwd(**kw) == code
    assert tfla.tfla_last_error()


def test_injected_allocation_failure(L, set_knob):
    set_knob(tfla.KNOB_FAULT_ALLOC, 1)
    assert fwd() == OOM
    assert "injected" in tfla.tfla_last_error()
    assert L.tfla_dbg_states(K, V, IG, FG, WS, 2, 3, 300, 128, 256, 64, SIG | BF16, None) == OOM


def test_workspace_bytes(L):
    def a256(x):
        return (x + 255) // 256 * 256

    # T = 250, L = 64: four chunks, too few to split the state walk into segments
    B, H, T, dqk, dhv, Lc = 2, 3, 250, 128, 256, 64
    nc = -(-T // Lc)
    # the states are stored in the I/O type: 2 bytes per element for bf16, 4 for fp32
    sig = a256(B * H * T * 4) * 2 + a256(B * H * nc * 4) + a256(B * H * (nc - 1) * dhv * dqk * 2)
    assert tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16) == sig
    sig32 = a256(B * H * T * 4) * 2 + a256(B * H * nc * 4) + a256(B * H * (nc - 1) * dhv * dqk * 4)
    assert tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG) == sig32
    scal = a256(B * H * (nc - 1) * dhv * dqk * 2)
    assert tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SCALAR | BF16) == scal
    # per-channel gate: a and g per key channel, and the walk's weighted keys in the I/O type
    gla = a256(B * H * T * dqk * 4) + a256(B * H * nc * dqk * 4) + a256(B * H * T * dqk * 2) + scal
    assert tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, GLA | BF16) == gla
    assert tfla.tfla_workspace_bytes(B, H, 64, dqk, dhv, Lc, SCALAR | BF16) == 0   # one chunk, no state
    # TFLA_STATES_FP32 (0x400): fp32 states with bf16 I/O; no effect with fp32 I/O
    assert tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16 | 0x400) == sig32
    assert tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | 0x400) == sig32
    assert tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16 | 0x800) == 0   # unknown flag
    assert tfla.tfla_workspace_bytes(B, H, T, 96, dhv, Lc, SIG) == 0


def test_segmented_state_walk_workspace(L):
    """A long chunk chain over few heads splits the state walk into P >= 2
    segments, whose start and end states ([B*H, P, d_qk, d_hv] fp32 each)
    join the workspace."""
    B, H, dqk, dhv, Lc = 1, 2, 128, 128, 64
    base = tfla.tfla_workspace_bytes(B, H, 250, dqk, dhv, Lc, SIG | BF16)        # 4 chunks: no segments
    T = 64 * 40
    nc = 40
    plain = (T * 4 * 2 + 256) + (nc * 4 + 256) + (nc - 1) * dhv * dqk * 2 * B * H
    seg = tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16)
    assert base > 0 and seg >= plain + 2 * B * H * 2 * dqk * dhv * 4


def test_fwd_ws_checks_workspace(L):
    need = tfla.tfla_workspace_bytes(2, 3, 300, 128, 256, 64, SIG | BF16)
    rc = L.tfla_fwd_ws(Q, K, V, IG, FG, H_, 2, 3, 300, 128, 256, 64, SIG | BF16, WS, need - 1, None)
    assert rc == OOM
    rc = L.tfla_fwd_ws(Q, K, V, IG, FG, H_, 2, 3, 300, 128, 256, 64, SIG | BF16, None, need, None)
    assert rc == INVALID
    rc = L.tfla_fwd_ws(Q, K, V, IG, FG, H_, 2, 3, 300, 128, 256, 64, SIG | BF16, WS + 16, need, None)
    assert rc == INVALID


def test_python_binding_raises(L):
    with pytest.raises(tfla.TflaError) as ei:
        tfla.tfla_fwd(Q, K, V, IG, FG, H_, 2, 3, 300, 96, 256, 64, SIG | BF16, stream=0)
    assert ei.value.code == UNSUPPORTED


def fwd_state(c0=C0, cf=CF, ws=WS, nws=1 << 30, **kw):
    a = dict(q=Q, k=K, v=V, ig=IG, fg=FG, h=H_, B=2, H=3, T=300, dqk=128, dhv=256, Lc=64, variant=SIG | BF16)
    a.update(kw)
    return tfla.lib().tfla_fwd_state(a["q"], a["k"], a["v"], a["ig"], a["fg"], c0, a["h"], cf, a["B"], a["H"],
                                     a["T"], a["dqk"], a["dhv"], a["Lc"], a["variant"], ws, nws, None)


SBYTES = 2 * 3 * 128 * 256 * 4   # one state per head at the shapes above


@pytest.mark.parametrize("kw,code", [
    (dict(c0=C0 + 4), INVALID), (dict(cf=CF + 8), INVALID),          # misaligned
    (dict(cf=H_ + 64), INVALID), (dict(c0=Q), INVALID),              # overlaps an input / h
    (dict(c0=K + 4096), INVALID), (dict(cf=FG), INVALID),
    (dict(cf=C0 + 256), INVALID),                                    # partial overlap of c0 and c_final
    (dict(nws=1000), OOM), (dict(ws=WS + 16), INVALID),               # workspace too small / misaligned
    (dict(dqk=96), UNSUPPORTED), (dict(q=None), INVALID), (dict(variant=7), INVALID),
])
def test_fwd_state_rejects_bad_arguments(L, kw, code):
    assert fwd_state(**kw) == code
    assert tfla.tfla_last_error()


def test_fwd_state_allocation_failure(L, set_knob):
    set_knob(tfla.KNOB_FAULT_ALLOC, 1)
    assert fwd_state(ws=None, nws=0) == OOM
    assert "injected" in tfla.tfla_last_error()


def test_state_workspace_bytes(L):
    def a256(x):
        return (x + 255) // 256 * 256

    B, H, T, dqk, dhv, Lc = 2, 3, 250, 128, 256, 64   # four chunks: no segmented state walk
    nc = -(-T // Lc)
    base = tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16)
    sig = a256(B * H * T * 4) * 2 + a256(B * H * nc * 4) + a256(B * H * nc * dhv * dqk * 2)
    assert tfla.tfla_state_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16) == sig > base
    # one chunk: the only state slot is the initial state's (bf16 like the I/O)
    assert tfla.tfla_state_workspace_bytes(B, H, 64, dqk, dhv, Lc, SCALAR | BF16) == a256(B * H * dhv * dqk * 2)
    assert tfla.tfla_state_workspace_bytes(B, H, T, 96, dhv, Lc, SIG) == 0


def rec(state=C0, **kw):
    a = dict(q=Q, k=K, v=V, ig=IG, fg=FG, h=H_, B=2, H=3, T=5, dqk=128, dhv=256, variant=SIG | BF16)
    a.update(kw)
    return tfla.lib().tfla_fwd_recurrent(a["q"], a["k"], a["v"], a["ig"], a["fg"], state, a["h"], a["B"], a["H"],
                                         a["T"], a["dqk"], a["dhv"], a["variant"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(state=None), INVALID), (dict(state=C0 + 4), INVALID), (dict(state=H_), INVALID),
    (dict(state=V + 256), INVALID), (dict(T=0), INVALID), (dict(ig=None), INVALID),
    (dict(dhv=100), UNSUPPORTED), (dict(dqk=512, variant=SIG), UNSUPPORTED),
])
def test_recurrent_rejects_bad_arguments(L, kw, code):
    assert rec(**kw) == code
    assert tfla.tfla_last_error()


# ---- backward entry point
DH, DQ, DK, DV, DIG, DFG = (0x10000000 * (n + 10) for n in range(6))


def bwd(q=Q, k=K, v=V, ig=IG, fg=FG, dh=DH, dq=DQ, dk=DK, dv=DV, dig=DIG, dfg=DFG, B=2, H=3, T=300, dqk=128,
        dhv=256, Lc=64, variant=SIG | BF16, ws=None, nws=0):
    return tfla.lib().tfla_bwd(q, k, v, ig, fg, dh, dq, dk, dv, dig, dfg, B, H, T, dqk, dhv, Lc, variant, ws, nws,
                               None)


@pytest.mark.parametrize("kw,code", [
    (dict(variant=GLA | BF16), INVALID),                          # per-channel gate: no input gate
    (dict(dhv=192), UNSUPPORTED), (dict(dhv=320), UNSUPPORTED),   # d_hv is contracted: powers of two
    (dict(variant=SIG, dhv=384), UNSUPPORTED),                    # fp32 I/O too
    (dict(dqk=96), UNSUPPORTED), (dict(Lc=32), UNSUPPORTED),
    (dict(B=0), INVALID), (dict(variant=7), INVALID),
    (dict(variant=SIG | BF16 | 0x400), UNSUPPORTED),               # TFLA_STATES_FP32: forward calls only
    (dict(dh=None), INVALID), (dict(dq=None), INVALID), (dict(dv=None), INVALID),
    (dict(dk=DK + 8), INVALID), (dict(dfg=None), INVALID), (dict(dfg=DFG + 2), INVALID),
    (dict(dig=None), INVALID),                                    # mLSTMsig needs dig
    (dict(variant=SCALAR | BF16, ig=None), INVALID),              # ... the others must not have one
    (dict(dq=Q + 64), INVALID), (dict(dv=DH), INVALID),           # an output overlaps an input
    (dict(dk=DQ + 16), INVALID), (dict(dig=DFG), INVALID),        # outputs overlap each other
    (dict(ws=WS + 16, nws=1 << 30), INVALID), (dict(ws=WS, nws=16), OOM),
])
def test_bwd_rejects_bad_arguments(L, kw, code):
    assert bwd(**kw) == code
    assert tfla.tfla_last_error()


def test_bwd_reuse_needs_the_forward_workspace(L):
    assert bwd(variant=SIG | BF16 | 0x200) == INVALID
    assert "workspace" in tfla.tfla_last_error()
    assert bwd(variant=SIG | BF16 | 0x800) == INVALID          # unknown flag
    n = tfla.tfla_bwd_workspace_bytes(2, 3, 300, 128, 256, 64, SIG | BF16)
    assert n > 0 and tfla.tfla_bwd_workspace_bytes(2, 3, 300, 128, 256, 64, SIG | BF16 | 0x200) == n


def test_bwd_injected_allocation_failure(L, set_knob):
    set_knob(tfla.KNOB_FAULT_ALLOC, 1)
    assert bwd() == OOM


def test_bwd_workspace_bytes(L):
    def a256(x):
        return (x + 255) // 256 * 256

    B, H, T, dqk, dhv, Lc = 2, 3, 250, 128, 256, 64
    nc = -(-T // Lc)
    states = a256(B * H * (nc - 1) * dhv * dqk * 2)   # reverse-walk states, I/O type
    steps = a256(B * H * T * 4)
    # forward workspace, reverse-walk states, mirrored gates (2), the row
    # partials of q.dq and k.dk (one per 128-wide tile of d_qk here), and
    # the partials of the coupling across each chunk boundary (64x64 state
    # tiles at this size, four waves each)
    X = a256(B * H * (nc - 1) * (dhv // 64) * (dqk // 64) * 4 * 4)
    sig = tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16) + states + 4 * steps + X
    assert tfla.tfla_bwd_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16) == sig
    scal = tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SCALAR | BF16) + states + 2 * steps + X + a256(B * H * 8)
    assert tfla.tfla_bwd_workspace_bytes(B, H, T, dqk, dhv, Lc, SCALAR | BF16) == scal
    # per-channel gate: mirrored gate exponents and per-element products per key channel,
    # coupling partials per key channel (value tiles x 2 row groups of 64x64 state tiles)
    Xg = a256(B * H * (nc - 1) * dqk * (dhv // 64) * 2 * 4)
    gla = (tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, GLA | BF16) + states + 3 * a256(B * H * T * dqk * 4)
           + Xg)
    assert tfla.tfla_bwd_workspace_bytes(B, H, T, dqk, dhv, Lc, GLA | BF16) == gla
    assert tfla.tfla_bwd_workspace_bytes(B, H, T, dqk, 192, Lc, SIG | BF16) == 0
    assert tfla.tfla_bwd_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16 | 0x400) == 0   # forward-only flag


def test_workspace_must_not_overlap_a_tensor(L):
    """Each workspace-taking entry point rejects a workspace that shares
    bytes with one of its tensors, before any HIP call."""
    B, H, T, dqk, dhv, Lc, var = 2, 3, 300, 128, 256, 64, SIG | BF16
    need = tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, var)
    assert L.tfla_fwd_ws(Q, K, V, IG, FG, H_, B, H, T, dqk, dhv, Lc, var, Q - 256, need, None) == INVALID
    assert "overlaps" in tfla.tfla_last_error()
    assert L.tfla_fwd_ws(Q, K, V, IG, FG, H_, B, H, T, dqk, dhv, Lc, var, H_ + 4096, need, None) == INVALID
    sneed = tfla.tfla_state_workspace_bytes(B, H, T, dqk, dhv, Lc, var)
    assert L.tfla_fwd_state(Q, K, V, IG, FG, C0, H_, CF, B, H, T, dqk, dhv, Lc, var, C0, sneed, None) == INVALID
    bneed = tfla.tfla_bwd_workspace_bytes(B, H, T, dqk, dhv, Lc, var)
    assert bwd(ws=DQ, nws=bneed) == INVALID
    assert bwd(ws=DIG, nws=bneed) == INVALID
    assert bwd(ws=FG - 256 * 256, nws=bneed) == INVALID


def bwd_state(c0=C0, dcf=CF, dc0=WS, variant=SIG | BF16, ws=None, nws=0, **kw):
    a = dict(q=Q, k=K, v=V, ig=IG, fg=FG, dh=DH, dq=DQ, dk=DK, dv=DV, dig=DIG, dfg=DFG)
    a.update(kw)
    return tfla.lib().tfla_bwd_state(a["q"], a["k"], a["v"], a["ig"], a["fg"], c0, a["dh"], dcf, a["dq"], a["dk"],
                                     a["dv"], a["dig"], a["dfg"], dc0, 2, 3, 300, 128, 256, 64, variant, ws, nws, None)


@pytest.mark.parametrize("kw,code", [
    (dict(c0=C0 + 8), INVALID), (dict(dc0=WS + 4), INVALID),            # misaligned state buffers
    (dict(dc0=DQ), INVALID), (dict(c0=DH + 64), INVALID),               # overlap a tensor
    (dict(dc0=C0 + 256), INVALID),                                      # partial overlap of c0
    (dict(dcf=C0 + 16), INVALID),                                       # c0 and dc_final overlap
    (dict(variant=SIG | BF16 | 0x200, ws=0x7000000000, nws=1 << 34), INVALID),  # no forward reuse here
    (dict(dhv=0), INVALID),
])
def test_bwd_state_rejects_bad_arguments(L, kw, code):
    if "dhv" in kw:
        assert tfla.lib().tfla_bwd_state(Q, K, V, IG, FG, C0, DH, CF, DQ, DK, DV, DIG, DFG, WS, 2, 3, 300, 128, 0, 64,
                                         SIG | BF16, None, 0, None) == code
        return
    assert bwd_state(**kw) == code
    assert tfla.tfla_last_error()


def test_bwd_state_workspace_bytes(L):
    a = tfla.tfla_bwd_workspace_bytes(2, 3, 250, 128, 256, 64, SIG | BF16)
    b = tfla.tfla_bwd_state_workspace_bytes(2, 3, 250, 128, 256, 64, SIG | BF16)
    assert b > a > 0
    assert tfla.tfla_bwd_state_workspace_bytes(2, 3, 250, 128, 192, 64, SIG | BF16) == 0


# ---- the binding checks tensors before a pointer reaches the library --------
def _cpu_case(gate=SIG, dtype=None, B=1, H=2, T=40, dqk=64, dhv=128):
    import torch
    dtype = dtype or torch.bfloat16
    q = torch.zeros(B, H, T, dqk, dtype=dtype)
    k = torch.zeros(B, H, T, dqk, dtype=dtype)
    v = torch.zeros(B, H, T, dhv, dtype=dtype)
    if gate == SIG:
        ig, fg = torch.zeros(B, H, T), torch.zeros(B, H, T)
    elif gate == SCALAR:
        ig, fg = None, torch.zeros(H)
    else:
        ig, fg = None, torch.zeros(B, H, T, dqk)
    return q, k, v, ig, fg


def _malformed():
    """(description, mutate(case) -> case, expected exception)"""
    import torch
    return [
        ("k transposed view", lambda c: (c[0], c[1].transpose(2, 3).contiguous().transpose(2, 3), *c[2:]), ValueError),
        ("v non-contiguous", lambda c: (c[0], c[1], torch.zeros(1, 2, 128, 40, dtype=c[2].dtype).transpose(2, 3),
                                         *c[3:]), ValueError),
        ("v of another dtype", lambda c: (c[0], c[1], c[2].float(), *c[3:]), TypeError),
        ("bf16 gate", lambda c: (*c[:3], c[3].to(torch.bfloat16), c[4]), TypeError),
        ("fgate of the wrong rank", lambda c: (*c[:4], c[4][..., None].expand(1, 2, 40, 64).contiguous()), ValueError),
        ("k of another length", lambda c: (c[0], c[1][:, :, :39].contiguous(), *c[2:]), ValueError),
        ("missing input gate", lambda c: (*c[:3], None, c[4]), ValueError),
    ]


@pytest.mark.parametrize("idx", range(7))
def test_binding_rejects_malformed_tensors(L, idx):
    name, mutate, exc = _malformed()[idx]
    q, k, v, ig, fg = mutate(_cpu_case())
    with pytest.raises(exc):
        tfla.forward(q, k, v, ig, fg, tfla.MLSTM_SIG, 64)
    import torch
    dh = torch.zeros(1, 2, 40, 128, dtype=torch.bfloat16)
    with pytest.raises(exc):
        tfla.backward(q, k, v, ig, fg, dh, tfla.MLSTM_SIG, 64)


def test_binding_rejects_gla_gate_shapes_and_cpu_tensors(L):
    import torch
    q, k, v, ig, fg = _cpu_case(GLA)
    with pytest.raises(ValueError):            # [B,H,T] is the per-step shape, not the per-channel one
        tfla.forward(q, k, v, None, fg[..., 0].contiguous(), tfla.GLA_KEY, 64)
    with pytest.raises(ValueError):            # an input gate where the variant has none
        tfla.forward(q, k, v, torch.zeros(1, 2, 40), fg, tfla.GLA_KEY, 64)
    q, k, v, ig, fg = _cpu_case(SCALAR)
    with pytest.raises(ValueError):            # fixed decay takes one logit per head
        tfla.forward(q, k, v, None, torch.zeros(1, 2, 40), tfla.SCALAR_DECAY, 64)
    with pytest.raises(ValueError, match="GPU memory"):   # well formed, but host tensors
        tfla.forward(q, k, v, None, fg, tfla.SCALAR_DECAY, 64)
    st = torch.zeros(1, 2, 64, 128)
    with pytest.raises(ValueError):            # state of the wrong orientation
        tfla.tfla_fwd_recurrent(q, k, v, None, fg, st.transpose(2, 3).contiguous(), torch.zeros_like(v),
                                1, 2, 40, 64, 128, SCALAR | BF16)
    with pytest.raises(ValueError):            # workspace smaller than the byte count passed
        tfla.tfla_fwd_ws(q, k, v, None, fg, torch.zeros_like(v), 1, 2, 40, 64, 128, 64, SCALAR | BF16,
                         torch.zeros(16, dtype=torch.uint8), 1024)


def test_knobs_are_set_and_cleared_through_the_hook(L, set_knob):
    assert L.tfla_dbg_set_knob(99, 1) == INVALID
    assert "knob" in tfla.tfla_last_error()
    assert L.tfla_dbg_set_knob(-1, 1) == INVALID
    # the segment knob changes the workspace the segmented walk needs
    B, H, T, dqk, dhv, Lc = 1, 2, 64 * 11 + 29, 64, 128, 64
    base = tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16)
    set_knob(tfla.KNOB_STATE_SEGMENTS, 2)            # by default this shape takes 4 segments
    assert tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16) < base
    set_knob(tfla.KNOB_STATE_SEGMENTS, 1)            # no segmented walk at all
    assert tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16) < base
    tfla.tfla_dbg_set_knob(tfla.KNOB_STATE_SEGMENTS, -1)
    assert tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16) == base


def test_noalloc_rejects_oversized_problems_before_any_hip_call(L):
    var = SIG | BF16
    need = tfla.tfla_workspace_bytes(4, 8, 8192, 256, 512, 64, var)
    assert need > L.tfla_fwd_noalloc_max_workspace() == 64 << 20
    rc = L.tfla_fwd_noalloc(Q, K, V, IG, FG, H_, 4, 8, 8192, 256, 512, 64, var, None)
    assert rc == OOM
    assert "scratch" in tfla.tfla_last_error()
    assert L.tfla_fwd_noalloc(Q, K, V, IG, FG, H_, 4, 8, 8192, 96, 512, 64, var, None) == UNSUPPORTED



def test_mlstm_exp_is_forward_only(L):
    """mLSTMexp has tfla_fwd / _ws / _noalloc only: the state-I/O, step-by-step
    and backward entry points and the test hooks reject it before any HIP
    call; its forward workspace holds the stabilised exponents, the lower
    bounds, the max-state chain and the normaliser states."""
    var = EXP | BF16
    B, H, T, dqk, dhv, Lc = 2, 3, 300, 128, 256, 64
    assert L.tfla_fwd_state(Q, K, V, IG, FG, None, H_, None, B, H, T, dqk, dhv, Lc, var, None, 0, None) == UNSUPPORTED
    assert "mLSTMexp" in tfla.tfla_last_error()
    assert L.tfla_fwd_recurrent(Q, K, V, IG, FG, C0, H_, B, H, T, dqk, dhv, var, None) == UNSUPPORTED
    assert L.tfla_bwd(Q, K, V, IG, FG, H_, WS, C0, CF, IG, FG, B, H, T, dqk, dhv, Lc, var, None, 0, None) == UNSUPPORTED
    assert tfla.tfla_bwd_workspace_bytes(B, H, T, dqk, dhv, Lc, var) == 0
    assert tfla.tfla_state_workspace_bytes(B, H, T, dqk, dhv, Lc, var) == 0
    assert L.tfla_dbg_gates(IG, FG, WS, C0, CF, B, H, T, dqk, Lc, var, None) == UNSUPPORTED
    assert L.tfla_dbg_states(K, V, IG, FG, WS, B, H, T, dqk, dhv, Lc, var, None) == UNSUPPORTED
    a256 = lambda n: (n + 255) // 256 * 256
    nc = -(-T // Lc)
    sig = tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, SIG | BF16)
    extra = a256(B * H * T * 4) + a256(B * H * nc * dqk * 4) + a256(B * H * (nc - 1) * dqk * 4) + 2 * a256(B * H * nc * 4)
    assert tfla.tfla_workspace_bytes(B, H, T, dqk, dhv, Lc, var) == sig + extra


def test_stream_probe_rejects_bad_arguments(L):
    """The streaming probe (a measurement aid) checks its arguments before
    any HIP call."""
    assert L.tfla_dbg_stream(2, Q, K, 1 << 20, 4, 256, None) == INVALID      # no such mode
    assert L.tfla_dbg_stream(0, Q, K, 1 << 20, 3, 256, None) == INVALID      # 3 loads per thread
    assert L.tfla_dbg_stream(0, Q, K, 1 << 20, 4, 0, None) == INVALID        # no workgroups
    assert L.tfla_dbg_stream(1, Q, K, 1000, 4, 256, None) == INVALID         # not a multiple of 16
    assert L.tfla_dbg_stream(0, Q + 8, K, 1 << 20, 4, 256, None) == INVALID  # misaligned
    assert L.tfla_dbg_stream(0, None, K, 1 << 20, 4, 256, None) == INVALID
    assert "tfla_dbg_stream" in tfla.tfla_last_error()


def test_mfma_probe_rejects_bad_arguments(L):
    """The matrix-core probe (a measurement aid) checks its arguments before
    any HIP call."""
    assert L.tfla_dbg_mfma(0, 256, Q, None) == INVALID        # no iterations
    assert L.tfla_dbg_mfma(100, 0, Q, None) == INVALID        # no workgroups
    assert L.tfla_dbg_mfma(100, 256, None, None) == INVALID   # no sink
    assert L.tfla_dbg_mfma(100, 256, Q + 8, None) == INVALID  # misaligned sink
    assert "tfla_dbg_mfma" in tfla.tfla_last_error()


def test_lds_probe_rejects_bad_arguments(L):
    """The LDS probe (a measurement aid) checks its arguments before any HIP
    call."""
    assert L.tfla_dbg_lds(5, 8, 100, 256, Q, K, None) == INVALID       # no such mode
    assert L.tfla_dbg_lds(0, 6, 100, 256, Q, K, None) == INVALID       # 6 waves
    assert L.tfla_dbg_lds(0, 8, 0, 256, Q, K, None) == INVALID         # no iterations
    assert L.tfla_dbg_lds(0, 8, 100, 0, Q, K, None) == INVALID         # no workgroups
    assert L.tfla_dbg_lds(0, 8, 100, 256, None, K, None) == INVALID    # no clock buffer
    assert L.tfla_dbg_lds(0, 8, 100, 256, Q + 4, K, None) == INVALID   # misaligned clock buffer
    assert L.tfla_dbg_lds(0, 8, 100, 256, Q, K + 8, None) == INVALID   # misaligned sink
    assert "tfla_dbg_lds" in tfla.tfla_last_error()

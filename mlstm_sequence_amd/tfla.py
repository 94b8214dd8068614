"""Thin ctypes binding of libtfla (include/tfla.h).

Argument marshalling only: torch tensors are passed as raw device pointers
and torch's current HIP stream as the stream; every step of the forward path
runs in the library's HIP kernels.  There is no fallback: when libtfla.so is
missing or a call fails, these functions raise.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first: libtfla then shares torch's HIP runtime (same SONAME)

MLSTM_SIG = 0
SCALAR_DECAY = 1
GLA_KEY = 2
IO_BF16 = 0x100
BWD_REUSE_FWD = 0x200
STATES_FP32 = 0x400   # forward, bf16 I/O: materialise the chunk states in fp32

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_OUT_OF_MEMORY = 0, 1, 2, 3, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtfla.so")
_lib = None


class TflaError(RuntimeError):
    def __init__(self, code: int, fn: str, detail: str):
        self.code = code
        super().__init__(f"{fn} failed ({code}: {error_string(code)}): {detail}")


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with mlstm_sequence_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, fp, i, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.tfla_fwd.argtypes = [vp, vp, vp, fp, fp, vp] + [i] * 7 + [vp]
        L.tfla_fwd.restype = i
        L.tfla_fwd_ws.argtypes = [vp, vp, vp, fp, fp, vp] + [i] * 7 + [vp, sz, vp]
        L.tfla_fwd_ws.restype = i
        L.tfla_fwd_ws_marked.argtypes = [vp, vp, vp, fp, fp, vp] + [i] * 7 + [vp, sz, vp, vp]
        L.tfla_fwd_ws_marked.restype = i
        L.tfla_workspace_bytes.argtypes = [i] * 7
        L.tfla_workspace_bytes.restype = sz
        L.tfla_fwd_state.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp] + [i] * 7 + [vp, sz, vp]
        L.tfla_fwd_state.restype = i
        L.tfla_state_workspace_bytes.argtypes = [i] * 7
        L.tfla_state_workspace_bytes.restype = sz
        L.tfla_fwd_recurrent.argtypes = [vp, vp, vp, fp, fp, fp, vp] + [i] * 6 + [vp]
        L.tfla_fwd_recurrent.restype = i
        L.tfla_bwd.argtypes = [vp, vp, vp, fp, fp, vp, vp, vp, vp, fp, fp] + [i] * 7 + [vp, sz, vp]
        L.tfla_bwd.restype = i
        L.tfla_bwd_workspace_bytes.argtypes = [i] * 7
        L.tfla_bwd_workspace_bytes.restype = sz
        L.tfla_bwd_state.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp, vp, vp, fp, fp, fp] + [i] * 7 + [vp, sz, vp]
        L.tfla_bwd_state.restype = i
        L.tfla_bwd_state_workspace_bytes.argtypes = [i] * 7
        L.tfla_bwd_state_workspace_bytes.restype = sz
        L.tfla_dbg_gates.argtypes = [fp, fp, fp, fp, fp] + [i] * 6 + [vp]
        L.tfla_dbg_gates.restype = i
        L.tfla_dbg_states.argtypes = [vp, vp, fp, fp, vp] + [i] * 7 + [vp]
        L.tfla_dbg_states.restype = i
        L.tfla_error_string.argtypes = [i]
        L.tfla_error_string.restype = ctypes.c_char_p
        L.tfla_last_error.argtypes = []
        L.tfla_last_error.restype = ctypes.c_char_p
        L.tfla_version.argtypes = []
        L.tfla_version.restype = i
        _lib = L
    return _lib


def error_string(code: int) -> str:
    return lib().tfla_error_string(code).decode()


def tfla_last_error() -> str:
    return lib().tfla_last_error().decode()


def tfla_version() -> int:
    return lib().tfla_version()


def _check(rc: int, fn: str):
    if rc != OK:
        raise TflaError(rc, fn, tfla_last_error())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def variant_of(gate: int, dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return gate | IO_BF16
    if dtype == torch.float32:
        return gate
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {dtype}")


def tfla_workspace_bytes(B, H, T, d_qk, d_hv, L, variant) -> int:
    return lib().tfla_workspace_bytes(B, H, T, d_qk, d_hv, L, variant)


def tfla_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, variant, stream=None):
    """tfla_fwd(...) of include/tfla.h on torch tensors (or raw pointers)."""
    rc = lib().tfla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(h),
                        B, H, T, d_qk, d_hv, L, variant, _stream(stream))
    _check(rc, "tfla_fwd")


def tfla_fwd_ws(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, variant, workspace,
                workspace_bytes, stream=None):
    rc = lib().tfla_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(h),
                           B, H, T, d_qk, d_hv, L, variant, _ptr(workspace), workspace_bytes,
                           _stream(stream))
    _check(rc, "tfla_fwd_ws")


def tfla_fwd_ws_marked(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, variant, workspace,
                       workspace_bytes, marks, stream=None):
    """``marks``: four raw hipEvent_t handles (ints), or None."""
    arr = None
    if marks is not None:
        arr = (ctypes.c_void_p * 4)(*marks)
    rc = lib().tfla_fwd_ws_marked(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(h),
                                  B, H, T, d_qk, d_hv, L, variant, _ptr(workspace), workspace_bytes, arr,
                                  _stream(stream))
    _check(rc, "tfla_fwd_ws_marked")


def tfla_state_workspace_bytes(B, H, T, d_qk, d_hv, L, variant) -> int:
    return lib().tfla_state_workspace_bytes(B, H, T, d_qk, d_hv, L, variant)


def tfla_fwd_state(q, k, v, igate_pre, fgate_pre, c0, h, c_final, B, H, T, d_qk, d_hv, L, variant,
                   workspace=None, workspace_bytes=0, stream=None):
    """tfla_fwd_state(...): c0 / c_final fp32 [B,H,d_qk,d_hv] or None;
    workspace None lets the library allocate it."""
    rc = lib().tfla_fwd_state(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(c0), _ptr(h),
                              _ptr(c_final), B, H, T, d_qk, d_hv, L, variant, _ptr(workspace),
                              workspace_bytes, _stream(stream))
    _check(rc, "tfla_fwd_state")


def tfla_fwd_recurrent(q, k, v, igate_pre, fgate_pre, state, h, B, H, T, d_qk, d_hv, variant, stream=None):
    """tfla_fwd_recurrent(...): ``state`` fp32 [B,H,d_qk,d_hv] is updated in place."""
    rc = lib().tfla_fwd_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(state),
                                  _ptr(h), B, H, T, d_qk, d_hv, variant, _stream(stream))
    _check(rc, "tfla_fwd_recurrent")


def tfla_bwd_workspace_bytes(B, H, T, d_qk, d_hv, L, variant) -> int:
    return lib().tfla_bwd_workspace_bytes(B, H, T, d_qk, d_hv, L, variant)


def tfla_bwd(q, k, v, igate_pre, fgate_pre, dh, dq, dk, dv, dig, dfg, B, H, T, d_qk, d_hv, L, variant,
             workspace=None, workspace_bytes=0, stream=None):
    """tfla_bwd(...): dq, dk, dv in the element type of q; dig (mLSTMsig,
    else None) and dfg fp32; workspace None lets the library allocate it."""
    rc = lib().tfla_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(dh), _ptr(dq),
                        _ptr(dk), _ptr(dv), _ptr(dig), _ptr(dfg), B, H, T, d_qk, d_hv, L, variant,
                        _ptr(workspace), workspace_bytes, _stream(stream))
    _check(rc, "tfla_bwd")


def tfla_bwd_state_workspace_bytes(B, H, T, d_qk, d_hv, L, variant) -> int:
    return lib().tfla_bwd_state_workspace_bytes(B, H, T, d_qk, d_hv, L, variant)


def tfla_bwd_state(q, k, v, igate_pre, fgate_pre, c0, dh, dc_final, dq, dk, dv, dig, dfg, dc0, B, H, T, d_qk, d_hv,
                   L, variant, workspace=None, workspace_bytes=0, stream=None):
    """tfla_bwd_state(...): c0, dc_final, dc0 fp32 [B,H,d_qk,d_hv] or None."""
    rc = lib().tfla_bwd_state(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(c0), _ptr(dh),
                              _ptr(dc_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dig), _ptr(dfg), _ptr(dc0),
                              B, H, T, d_qk, d_hv, L, variant, _ptr(workspace), workspace_bytes, _stream(stream))
    _check(rc, "tfla_bwd_state")


def tfla_dbg_gates(igate_pre, fgate_pre, a_out, li_out, g_out, B, H, T, d_qk, L, variant, stream=None):
    rc = lib().tfla_dbg_gates(_ptr(igate_pre), _ptr(fgate_pre), _ptr(a_out), _ptr(li_out), _ptr(g_out),
                              B, H, T, d_qk, L, variant, _stream(stream))
    _check(rc, "tfla_dbg_gates")


def tfla_dbg_states(k, v, igate_pre, fgate_pre, states_out, B, H, T, d_qk, d_hv, L, variant, stream=None):
    rc = lib().tfla_dbg_states(_ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(states_out),
                               B, H, T, d_qk, d_hv, L, variant, _stream(stream))
    _check(rc, "tfla_dbg_states")


# ---- tensor-level conveniences (still marshalling only) ----------------------

def _dims(q, v):
    B, H, T, d_qk = q.shape
    return B, H, T, d_qk, v.shape[-1]


def forward(q, k, v, igate_pre, fgate_pre, gate: int, L: int, h=None, workspace=None, stream=None):
    """Allocates h (unless given) and runs the forward path on device tensors.
    With ``workspace`` (a uint8 device tensor of at least
    tfla_workspace_bytes bytes) the allocation-free entry point is used."""
    B, H, T, d_qk, d_hv = _dims(q, v)
    var = variant_of(gate, q.dtype)
    if h is None:
        h = torch.empty((B, H, T, d_hv), dtype=q.dtype, device=q.device)
    if workspace is None:
        tfla_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, var, stream)
    else:
        tfla_fwd_ws(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, var, workspace,
                    workspace.numel() * workspace.element_size(), stream)
    return h


def backward(q, k, v, igate_pre, fgate_pre, dh, gate: int, L: int, workspace=None, stream=None):
    """Allocates the gradients and runs the backward path on device tensors;
    returns (dq, dk, dv, dig, dfg), dig None unless mLSTMsig."""
    B, H, T, d_qk, d_hv = _dims(q, v)
    var = variant_of(gate, q.dtype)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dig = torch.empty_like(igate_pre) if igate_pre is not None else None
    dfg = torch.empty_like(fgate_pre)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    tfla_bwd(q, k, v, igate_pre, fgate_pre, dh, dq, dk, dv, dig, dfg, B, H, T, d_qk, d_hv, L, var,
             workspace, nbytes, stream)
    return dq, dk, dv, dig, dfg


def workspace_for(q, v, gate: int, L: int) -> torch.Tensor:
    B, H, T, d_qk, d_hv = _dims(q, v)
    n = tfla_workspace_bytes(B, H, T, d_qk, d_hv, L, variant_of(gate, q.dtype))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)

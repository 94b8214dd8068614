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
MLSTM_EXP = 3   # mLSTMexp: exponential input gate, normaliser and max state (forward only)
IO_BF16 = 0x100
BWD_REUSE_FWD = 0x200
STATES_FP32 = 0x400   # forward, bf16 I/O: materialise the chunk states in fp32

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_OUT_OF_MEMORY = 0, 1, 2, 3, 4

# test overrides (tfla_dbg_set_knob)
(KNOB_INTRA_SWEEP, KNOB_INTRA_BV, KNOB_INTRA_ROWS, KNOB_STATE_SEGMENTS, KNOB_STATE_SB, KNOB_FAULT_ALLOC,
 KNOB_STATE_REWALK) = range(7)

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
        L.tfla_fwd_noalloc.argtypes = [vp, vp, vp, fp, fp, vp] + [i] * 7 + [vp]
        L.tfla_fwd_noalloc.restype = i
        L.tfla_fwd_noalloc_max_workspace.argtypes = []
        L.tfla_fwd_noalloc_max_workspace.restype = sz
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
        L.tfla_dbg_stream.argtypes = [i, vp, vp, sz, i, i, vp]
        L.tfla_dbg_stream.restype = i
        L.tfla_dbg_mfma.argtypes = [i, i, vp, vp]
        L.tfla_dbg_mfma.restype = i
        L.tfla_dbg_lds.argtypes = [i, i, i, i, vp, vp, vp]
        L.tfla_dbg_lds.restype = i
        L.tfla_dbg_set_knob.argtypes = [i, i]
        L.tfla_dbg_set_knob.restype = i
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


def tfla_dbg_set_knob(which: int, value: int):
    """Test hook: set (value >= 0) or clear (value < 0) a process-wide override."""
    _check(lib().tfla_dbg_set_knob(which, value), "tfla_dbg_set_knob")


class knob:
    """Context manager: ``with tfla.knob(tfla.KNOB_STATE_SEGMENTS, 3): ...``
    sets the override for the block and clears it afterwards."""

    def __init__(self, which: int, value: int):
        self.which, self.value = which, value

    def __enter__(self):
        tfla_dbg_set_knob(self.which, self.value)
        return self

    def __exit__(self, *exc):
        tfla_dbg_set_knob(self.which, -1)
        return False


def _check(rc: int, fn: str):
    if rc != OK:
        raise TflaError(rc, fn, tfla_last_error())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


# ---- argument checks on tensors (before any pointer reaches the library) ------
#
# The library validates sizes, alignment and overlaps, but it cannot see a
# tensor's shape, strides, dtype or device: a transposed view, a bf16 gate
# or a gate of the wrong rank would make its kernels read past the end of a
# buffer.  Every tensor handed to an entry point is checked here first
# (raw integer pointers are the caller's responsibility).

def _io_dtype(variant: int):
    return torch.bfloat16 if variant & IO_BF16 else torch.float32


def _expect(t, name: str, shape, dtype, device=None, flat_ok=False):
    """Raises TypeError / ValueError unless ``t`` (a tensor, a raw pointer
    or None) is a contiguous tensor of exactly ``shape`` and ``dtype`` (on
    ``device`` when given); ``flat_ok``: any shape with that many elements
    (output buffers of the test hooks).  Returns the tensor's device."""
    if t is None or isinstance(t, int):
        return device
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, a raw device pointer or None, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    n = 1
    for x in shape:
        n *= x
    if (t.numel() != n) if flat_ok else (tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major), got strides {t.stride()}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, other tensors on {device}")
    return t.device


def _require_null(t, name: str, why: str):
    if t is not None:
        raise ValueError(f"{name} must be None: {why}")


def _check_device(dev):
    if dev is not None and dev.type != "cuda":
        raise ValueError(f"tensors must live in GPU memory, got {dev}")


def _check_gates(igate_pre, fgate_pre, B, H, T, d_qk, variant, dev, ig_name="igate_pre", fg_name="fgate_pre"):
    gate = variant & 0xFF
    if gate in (MLSTM_SIG, MLSTM_EXP):
        if igate_pre is None:
            raise ValueError(f"{ig_name} is required for mLSTMsig")
        dev = _expect(igate_pre, ig_name, (B, H, T), torch.float32, dev)
        return _expect(fgate_pre, fg_name, (B, H, T), torch.float32, dev)
    _require_null(igate_pre, ig_name, "this variant has no input gate")
    if gate == SCALAR_DECAY:
        return _expect(fgate_pre, fg_name, (H,), torch.float32, dev)
    return _expect(fgate_pre, fg_name, (B, H, T, d_qk), torch.float32, dev)


def _check_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, variant, extra=()):
    """q, k, v, h and the gates of a forward call; ``extra``: further
    (tensor, name, shape, dtype) to check on the same device."""
    io = _io_dtype(variant)
    dev = _expect(q, "q", (B, H, T, d_qk), io)
    dev = _expect(k, "k", (B, H, T, d_qk), io, dev)
    dev = _expect(v, "v", (B, H, T, d_hv), io, dev)
    dev = _expect(h, "h", (B, H, T, d_hv), io, dev)
    dev = _check_gates(igate_pre, fgate_pre, B, H, T, d_qk, variant, dev)
    for t, name, shape, dtype in extra:
        dev = _expect(t, name, shape, dtype, dev)
    _check_device(dev)
    return dev


def _check_workspace(ws, nbytes: int, dev):
    if ws is None or isinstance(ws, int):
        return
    if not isinstance(ws, torch.Tensor) or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace tensor holds {ws.numel() * ws.element_size()} bytes, {nbytes} were passed")
    if dev is not None and ws.device != dev:
        raise ValueError(f"workspace is on {ws.device}, tensors on {dev}")


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


def _check_bwd(q, k, v, igate_pre, fgate_pre, dh, dq, dk, dv, dig, dfg, B, H, T, d_qk, d_hv, variant, extra=()):
    io = _io_dtype(variant)
    dev = _check_fwd(q, k, v, igate_pre, fgate_pre, dh, B, H, T, d_qk, d_hv, variant)
    dev = _expect(dq, "dq", (B, H, T, d_qk), io, dev)
    dev = _expect(dk, "dk", (B, H, T, d_qk), io, dev)
    dev = _expect(dv, "dv", (B, H, T, d_hv), io, dev)
    dev = _check_gates(dig, dfg, B, H, T, d_qk, variant, dev, "dig", "dfg")
    for t, name, shape, dtype in extra:
        dev = _expect(t, name, shape, dtype, dev)
    _check_device(dev)
    return dev


def tfla_workspace_bytes(B, H, T, d_qk, d_hv, L, variant) -> int:
    return lib().tfla_workspace_bytes(B, H, T, d_qk, d_hv, L, variant)


def tfla_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, variant, stream=None):
    """tfla_fwd(...) of include/tfla.h on torch tensors (or raw pointers)."""
    _check_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, variant)
    rc = lib().tfla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(h),
                        B, H, T, d_qk, d_hv, L, variant, _stream(stream))
    _check(rc, "tfla_fwd")


def tfla_fwd_noalloc(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, variant, stream=None):
    """tfla_fwd_noalloc(...): tfla_fwd with the library's static scratch as
    workspace (no allocation; see include/tfla.h for its size limit)."""
    _check_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, variant)
    rc = lib().tfla_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(h),
                                B, H, T, d_qk, d_hv, L, variant, _stream(stream))
    _check(rc, "tfla_fwd_noalloc")


def tfla_fwd_noalloc_max_workspace() -> int:
    return lib().tfla_fwd_noalloc_max_workspace()


def tfla_fwd_ws(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, variant, workspace,
                workspace_bytes, stream=None):
    _check_workspace(workspace, workspace_bytes,
                     _check_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, variant))
    rc = lib().tfla_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(h),
                           B, H, T, d_qk, d_hv, L, variant, _ptr(workspace), workspace_bytes,
                           _stream(stream))
    _check(rc, "tfla_fwd_ws")


def tfla_fwd_ws_marked(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, L, variant, workspace,
                       workspace_bytes, marks, stream=None):
    """``marks``: four raw hipEvent_t handles (ints), or None."""
    _check_workspace(workspace, workspace_bytes,
                     _check_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, variant))
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
    st = (B, H, d_qk, d_hv)
    _check_workspace(workspace, workspace_bytes,
                     _check_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, variant,
                                [(c0, "c0", st, torch.float32), (c_final, "c_final", st, torch.float32)]))
    rc = lib().tfla_fwd_state(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(c0), _ptr(h),
                              _ptr(c_final), B, H, T, d_qk, d_hv, L, variant, _ptr(workspace),
                              workspace_bytes, _stream(stream))
    _check(rc, "tfla_fwd_state")


def tfla_fwd_recurrent(q, k, v, igate_pre, fgate_pre, state, h, B, H, T, d_qk, d_hv, variant, stream=None):
    """tfla_fwd_recurrent(...): ``state`` fp32 [B,H,d_qk,d_hv] is updated in place."""
    _check_fwd(q, k, v, igate_pre, fgate_pre, h, B, H, T, d_qk, d_hv, variant,
               [(state, "state", (B, H, d_qk, d_hv), torch.float32)])
    rc = lib().tfla_fwd_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(state),
                                  _ptr(h), B, H, T, d_qk, d_hv, variant, _stream(stream))
    _check(rc, "tfla_fwd_recurrent")


def tfla_bwd_workspace_bytes(B, H, T, d_qk, d_hv, L, variant) -> int:
    return lib().tfla_bwd_workspace_bytes(B, H, T, d_qk, d_hv, L, variant)


def tfla_bwd(q, k, v, igate_pre, fgate_pre, dh, dq, dk, dv, dig, dfg, B, H, T, d_qk, d_hv, L, variant,
             workspace=None, workspace_bytes=0, stream=None):
    """tfla_bwd(...): dq, dk, dv in the element type of q; dig (mLSTMsig,
    else None) and dfg fp32; workspace None lets the library allocate it."""
    _check_workspace(workspace, workspace_bytes,
                     _check_bwd(q, k, v, igate_pre, fgate_pre, dh, dq, dk, dv, dig, dfg, B, H, T, d_qk, d_hv,
                                variant))
    rc = lib().tfla_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(dh), _ptr(dq),
                        _ptr(dk), _ptr(dv), _ptr(dig), _ptr(dfg), B, H, T, d_qk, d_hv, L, variant,
                        _ptr(workspace), workspace_bytes, _stream(stream))
    _check(rc, "tfla_bwd")


def tfla_bwd_state_workspace_bytes(B, H, T, d_qk, d_hv, L, variant) -> int:
    return lib().tfla_bwd_state_workspace_bytes(B, H, T, d_qk, d_hv, L, variant)


def tfla_bwd_state(q, k, v, igate_pre, fgate_pre, c0, dh, dc_final, dq, dk, dv, dig, dfg, dc0, B, H, T, d_qk, d_hv,
                   L, variant, workspace=None, workspace_bytes=0, stream=None):
    """tfla_bwd_state(...): c0, dc_final, dc0 fp32 [B,H,d_qk,d_hv] or None."""
    st = (B, H, d_qk, d_hv)
    _check_workspace(workspace, workspace_bytes,
                     _check_bwd(q, k, v, igate_pre, fgate_pre, dh, dq, dk, dv, dig, dfg, B, H, T, d_qk, d_hv,
                                variant, [(c0, "c0", st, torch.float32), (dc_final, "dc_final", st, torch.float32),
                                          (dc0, "dc0", st, torch.float32)]))
    rc = lib().tfla_bwd_state(_ptr(q), _ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(c0), _ptr(dh),
                              _ptr(dc_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dig), _ptr(dfg), _ptr(dc0),
                              B, H, T, d_qk, d_hv, L, variant, _ptr(workspace), workspace_bytes, _stream(stream))
    _check(rc, "tfla_bwd_state")


def tfla_dbg_gates(igate_pre, fgate_pre, a_out, li_out, g_out, B, H, T, d_qk, L, variant, stream=None):
    nc = -(-T // L)
    w = (d_qk,) if (variant & 0xFF) == GLA_KEY else ()
    dev = _check_gates(igate_pre, fgate_pre, B, H, T, d_qk, variant, None)
    dev = _expect(a_out, "a_out", (B, H, T) + w, torch.float32, dev, flat_ok=True)
    dev = _expect(li_out, "li_out", (B, H, T), torch.float32, dev, flat_ok=True)
    _check_device(_expect(g_out, "g_out", (B, H, nc) + w, torch.float32, dev, flat_ok=True))
    rc = lib().tfla_dbg_gates(_ptr(igate_pre), _ptr(fgate_pre), _ptr(a_out), _ptr(li_out), _ptr(g_out),
                              B, H, T, d_qk, L, variant, _stream(stream))
    _check(rc, "tfla_dbg_gates")


def tfla_dbg_stream(mode, src, dst, nbytes, loads_per_thread, workgroups, stream=None):
    """Streaming probe (measurement aid): mode 0 reads ``nbytes`` of ``src``,
    mode 1 copies them to ``dst``; both CUDA tensors of at least ``nbytes``
    (``dst`` at least 4 KB in mode 0)."""
    for t, name in ((src, "src"), (dst, "dst")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA tensor")
    need = (nbytes, max(4096, nbytes if mode == 1 else 0))
    if src.numel() * src.element_size() < need[0] or dst.numel() * dst.element_size() < need[1]:
        raise ValueError("tfla_dbg_stream: buffers smaller than the bytes asked for")
    rc = lib().tfla_dbg_stream(mode, _ptr(src), _ptr(dst), nbytes, loads_per_thread, workgroups, _stream(stream))
    _check(rc, "tfla_dbg_stream")


def tfla_dbg_mfma(iters, workgroups, sink, stream=None):
    """Matrix-core probe (measurement aid): 4 * iters * 32768 flops per
    wavefront, 4 wavefronts per workgroup; ``sink`` a CUDA tensor of at
    least 1 KB."""
    if not isinstance(sink, torch.Tensor) or not sink.is_cuda:
        raise TypeError("sink must be a CUDA tensor")
    if sink.numel() * sink.element_size() < 1024:
        raise ValueError("tfla_dbg_mfma: sink smaller than 1 KB")
    _check(lib().tfla_dbg_mfma(iters, workgroups, _ptr(sink), _stream(stream)), "tfla_dbg_mfma")


def tfla_dbg_lds(mode, waves, iters, workgroups, clocks, sink, stream=None):
    """LDS probe (measurement aid): ``clocks`` an int64 CUDA tensor of at
    least 2 * workgroups elements (shader clock before / after each
    workgroup's loop), ``sink`` a CUDA tensor of at least 2 KB."""
    for name, t in (("clocks", clocks), ("sink", sink)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA tensor")
    if clocks.dtype != torch.int64 or clocks.numel() < 2 * workgroups:
        raise ValueError("tfla_dbg_lds: clocks must be int64 with 2 * workgroups elements")
    if sink.numel() * sink.element_size() < 2048:
        raise ValueError("tfla_dbg_lds: sink smaller than 2 KB")
    _check(lib().tfla_dbg_lds(mode, waves, iters, workgroups, _ptr(clocks), _ptr(sink), _stream(stream)),
           "tfla_dbg_lds")


def tfla_dbg_states(k, v, igate_pre, fgate_pre, states_out, B, H, T, d_qk, d_hv, L, variant, stream=None):
    io = _io_dtype(variant)
    st = torch.float32 if (variant & STATES_FP32 or io == torch.float32) else io
    nc = -(-T // L)
    dev = _expect(k, "k", (B, H, T, d_qk), io)
    dev = _expect(v, "v", (B, H, T, d_hv), io, dev)
    dev = _check_gates(igate_pre, fgate_pre, B, H, T, d_qk, variant, dev)
    if nc > 1:
        dev = _expect(states_out, "states_out", (B, H, nc - 1, d_hv, d_qk), st, dev)
    _check_device(dev)
    rc = lib().tfla_dbg_states(_ptr(k), _ptr(v), _ptr(igate_pre), _ptr(fgate_pre), _ptr(states_out),
                               B, H, T, d_qk, d_hv, L, variant, _stream(stream))
    _check(rc, "tfla_dbg_states")


# ---- tensor-level conveniences (still marshalling only) ----------------------

def _dims(q, v):
    if not isinstance(q, torch.Tensor) or not isinstance(v, torch.Tensor) or q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be 4-d tensors [B,H,T,d]")
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

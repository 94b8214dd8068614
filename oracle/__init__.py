"""CPU oracle for the gated linear-attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``mlstm_sequence_amd``) and never imports it.

Three independent evaluations of one function live here:

* :func:`recurrent_fwd` -- the step-by-step recurrence in double, in plain C
  (``oracle.c``, OpenMP over heads).  This is *the* oracle: the recurrent
  ("FusedRecurrent", O(T)) form listed among the computation forms of the
  flash-linear-attention README.
* :func:`closed_form_fwd` -- the quadratic closed form, brute force in numpy
  float64 (the "Parallel", O(T^2) form of the same README):
      h_t = sum_{s<=t} (prod_{r=s+1..t} f_r) i_s (q_t . k_s) v_s / sqrt(d_qk)
  with the product taken per key channel inside q.k for the per-channel gate.
* :func:`chunkwise_fwd` -- the chunkwise-parallel form ("ParallelChunk" in the
  README; the chunkwise formulation that Tiled Flash Linear Attention tiles,
  TFLA abstract) in numpy float64 for any chunk size, ragged last chunk
  included: an inter-chunk state recurrence plus a masked intra-chunk product.

The two numpy forms exist to pin the C oracle; they are slower and limited to
tiny inputs.  Gate variants (``kind``):

* 0 ``MLSTM_SIG``: i = sigmoid(igate_pre[t]), f = sigmoid(fgate_pre[t])
  (mLSTMsig: sigmoid input gate, no normaliser, no max state -- TFLA
  research-map summary, Approach).
* 1 ``SCALAR``: i = 1, f = sigmoid(fgate_pre[h]) per head (RetNet-style fixed
  decay, README model table).
* 2 ``GLA``: i = 1, f_{t,c} = exp(logsigmoid(x_{t,c}) / 16) per key channel
  (data-dependent gates, GLA abstract).

mLSTMexp (exponential input gate with normaliser and max state, the variant
mLSTMsig simplifies: TFLA research-map summary, Approach) has its own
recurrent oracle :func:`recurrent_fwd_exp`, pinned by
:func:`closed_form_fwd_exp` and :func:`chunkwise_fwd_exp`.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

MLSTM_SIG, SCALAR, GLA = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run oracle.build.build()")
        lib = ctypes.CDLL(LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_fwd.argtypes = [dp] * 7 + [ctypes.c_int] * 7
        lib.oracle_fwd.restype = ctypes.c_int
        lib.oracle_fwd_state.argtypes = [dp] * 9 + [ctypes.c_int] * 7
        lib.oracle_fwd_state.restype = ctypes.c_int
        lib.oracle_bwd.argtypes = [dp] * 11 + [ctypes.c_int] * 6
        lib.oracle_bwd.restype = ctypes.c_int
        lib.oracle_bwd_state.argtypes = [dp] * 14 + [ctypes.c_int] * 6
        lib.oracle_bwd_state.restype = ctypes.c_int
        lib.oracle_log_gates.argtypes = [dp] * 5 + [ctypes.c_int] * 6
        lib.oracle_log_gates.restype = ctypes.c_int
        lib.oracle_fwd_exp.argtypes = [dp] * 6 + [ctypes.c_int] * 5
        lib.oracle_fwd_exp.restype = ctypes.c_int
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_sigmoid.argtypes = [ctypes.c_double]
        lib.oracle_sigmoid.restype = ctypes.c_double
        lib.oracle_log_sigmoid.argtypes = [ctypes.c_double]
        lib.oracle_log_sigmoid.restype = ctypes.c_double
        _lib = lib
    return _lib


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def threads() -> int:
    """OpenMP threads the C oracle runs with."""
    return _load().oracle_threads()


def sigmoid(x: float) -> float:
    return _load().oracle_sigmoid(float(x))


def log_sigmoid(x: float) -> float:
    return _load().oracle_log_sigmoid(float(x))


def recurrent_fwd(q, k, v, igate_pre, fgate_pre, kind, L=None):
    """Recurrent oracle.  Arrays: q,k [B,H,T,dqk], v [B,H,T,dhv] (any real
    dtype; converted exactly to float64).  Returns h [B,H,T,dhv] float64, and
    with ``L`` also the states after every full block of L steps
    [B,H,T//L,dqk,dhv]."""
    q, k, v, ig, fg = map(_f64, (q, k, v, igate_pre, fgate_pre))
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    h = np.empty((B, H, T, dhv), dtype=np.float64)
    states = None
    if L is not None:
        states = np.empty((B, H, T // L, dqk, dhv), dtype=np.float64)
    rc = _load().oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(ig), _ptr(fg), _ptr(h),
                            _ptr(states), B, H, T, dqk, dhv, L or 0, kind)
    if rc != 0:
        raise ValueError("oracle_fwd rejected its arguments")
    return (h, states) if L is not None else h


def recurrent_fwd_exp(q, k, v, igate_pre, fgate_pre):
    """mLSTMexp oracle (``oracle_fwd_exp`` in oracle.c): exponential input
    gate exp(igate_pre), forget gate sigmoid(fgate_pre), normaliser state and
    max state, stepped in double.  Returns h [B,H,T,dhv] float64."""
    q, k, v, ig, fg = map(_f64, (q, k, v, igate_pre, fgate_pre))
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    h = np.empty((B, H, T, dhv), dtype=np.float64)
    rc = _load().oracle_fwd_exp(_ptr(q), _ptr(k), _ptr(v), _ptr(ig), _ptr(fg), _ptr(h), B, H, T, dqk, dhv)
    if rc != 0:
        raise ValueError("oracle_fwd_exp rejected its arguments")
    return h


def closed_form_fwd_exp(q, k, v, igate_pre, fgate_pre):
    """mLSTMexp by its plain definition, brute force in numpy float64 (no
    max state; overflows once exp(igate_pre) does):
        num_t = sum_{s<=t} (prod_{r=s+1..t} f_r) e^{igate_pre_s} (q_t . k_s) v_s / sqrt(d)
        den_t = the same sum without v_s
        h_t   = num_t / max(|den_t|, 1)"""
    q, k, v, ig, fg = map(_f64, (q, k, v, igate_pre, fgate_pre))
    B, H, T, dqk = q.shape
    f = 1.0 / (1.0 + np.exp(-fg))
    i = np.exp(ig)
    h = np.zeros(v.shape)
    for b in range(B):
        for hd in range(H):
            for t in range(T):
                num = np.zeros(v.shape[-1])
                den = 0.0
                for s_ in range(t + 1):
                    w = np.prod(f[b, hd, s_ + 1:t + 1]) * i[b, hd, s_] * np.dot(q[b, hd, t], k[b, hd, s_])
                    num += w * v[b, hd, s_]
                    den += w
                num /= np.sqrt(dqk)
                den /= np.sqrt(dqk)
                h[b, hd, t] = num / max(abs(den), 1.0)
    return h


def chunkwise_fwd_exp(q, k, v, igate_pre, fgate_pre, L):
    """mLSTMexp in chunkwise-parallel form, numpy float64, any chunk size L
    (ragged last chunk included), each chunk stabilised by its own running
    maximum: per chunk, the carried states (C, n) and their log scale m enter
    every row with weight e^{a_t + m}, the rows' own pairs with
    e^{a_t - a_s + igate_pre_s}; every term is taken relative to the row's
    largest log weight before exponentiating, and the carried states are
    renormalised to the largest log weight reaching the chunk's end."""
    q, k, v, ig, fg = map(_f64, (q, k, v, igate_pre, fgate_pre))
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    lf = np.minimum(fg, 0.0) - np.log1p(np.exp(-np.abs(fg)))
    h = np.zeros((B, H, T, dhv))
    sc = 1.0 / np.sqrt(dqk)
    for b in range(B):
        for hd in range(H):
            C = np.zeros((dqk, dhv))
            n = np.zeros(dqk)
            m = -np.inf                                   # log scale of (C, n)
            for t0 in range(0, T, L):
                t1 = min(t0 + L, T)
                a = np.cumsum(lf[b, hd, t0:t1])           # chunk-local log decay
                for t in range(t0, t1):
                    r = t - t0
                    logw = a[r] - a[:r + 1] + ig[b, hd, t0:t + 1]      # the chunk's pairs s <= t
                    top = max(a[r] + m, np.max(logw))
                    if top == -np.inf:
                        continue                            # nothing has entered: h_t = 0
                    w = np.exp(logw - top)
                    qk = k[b, hd, t0:t + 1] @ q[b, hd, t]
                    num = (w * qk) @ v[b, hd, t0:t + 1]
                    den = np.dot(w, qk)
                    if m != -np.inf:
                        ci = np.exp(a[r] + m - top)
                        num = num + ci * (q[b, hd, t] @ C)
                        den = den + ci * np.dot(q[b, hd, t], n)
                    h[b, hd, t] = num * sc / max(abs(den) * sc, np.exp(-top))
                # carry to the chunk end
                g = a[-1]
                logw = g - a + ig[b, hd, t0:t1]
                top = max(g + m, np.max(logw))
                if top == -np.inf:
                    C[:] = 0.0
                    n[:] = 0.0
                    m = -np.inf
                    continue
                w = np.exp(logw - top)
                cc = np.exp(g + m - top) if m != -np.inf else 0.0
                C = cc * C + (k[b, hd, t0:t1] * w[:, None]).T @ v[b, hd, t0:t1]
                n = cc * n + w @ k[b, hd, t0:t1]
                m = top
    return h


def recurrent_fwd_state(q, k, v, igate_pre, fgate_pre, kind, c0=None):
    """Recurrent oracle from an initial state C_0 = c0 ([B,H,dqk,dhv]; None
    means zero).  Returns (h [B,H,T,dhv], C_T [B,H,dqk,dhv])."""
    q, k, v, ig, fg, c0 = map(_f64, (q, k, v, igate_pre, fgate_pre, c0))
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    h = np.empty((B, H, T, dhv), dtype=np.float64)
    cT = np.empty((B, H, dqk, dhv), dtype=np.float64)
    rc = _load().oracle_fwd_state(_ptr(q), _ptr(k), _ptr(v), _ptr(ig), _ptr(fg), _ptr(c0), _ptr(h), None,
                                  _ptr(cT), B, H, T, dqk, dhv, 0, kind)
    if rc != 0:
        raise ValueError("oracle_fwd_state rejected its arguments")
    return h, cT


def recurrent_bwd(q, k, v, igate_pre, fgate_pre, dh, kind):
    """Reverse-mode derivative of the recurrence for the upstream gradient
    dh [B,H,T,dhv].  Returns (dq, dk, dv, dig, dfg): dig like igate_pre
    (None unless mLSTMsig), dfg like fgate_pre."""
    q, k, v, ig, fg, dh = map(_f64, (q, k, v, igate_pre, fgate_pre, dh))
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    dig = np.empty_like(ig) if kind == MLSTM_SIG else None
    dfg = np.empty_like(fg)
    rc = _load().oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(ig), _ptr(fg), _ptr(dh), _ptr(dq), _ptr(dk), _ptr(dv),
                            _ptr(dig), _ptr(dfg), B, H, T, dqk, dhv, kind)
    if rc != 0:
        raise ValueError("oracle_bwd rejected its arguments")
    return dq, dk, dv, dig, dfg


def recurrent_bwd_state(q, k, v, igate_pre, fgate_pre, dh, kind, c0=None, dcT=None):
    """The backward pass with an initial state C_0 = c0 [B,H,dqk,dhv] (None:
    0) and the gradient dcT of the loss with respect to the final state C_T
    (None: 0), i.e. for L = sum(dh * h) + sum(dcT * C_T).  Returns (dq, dk, dv,
    dig, dfg, dc0), dc0 = dL/dC_0."""
    q, k, v, ig, fg, dh, c0, dcT = map(_f64, (q, k, v, igate_pre, fgate_pre, dh, c0, dcT))
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    dig = np.empty_like(ig) if kind == MLSTM_SIG else None
    dfg = np.empty_like(fg)
    dc0 = np.empty((B, H, dqk, dhv), dtype=np.float64)
    rc = _load().oracle_bwd_state(_ptr(q), _ptr(k), _ptr(v), _ptr(ig), _ptr(fg), _ptr(c0), _ptr(dh), _ptr(dcT),
                                  _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dig), _ptr(dfg), _ptr(dc0),
                                  B, H, T, dqk, dhv, kind)
    if rc != 0:
        raise ValueError("oracle_bwd_state rejected its arguments")
    return dq, dk, dv, dig, dfg, dc0


def log_gates(igate_pre, fgate_pre, kind, B, H, T, dqk, L):
    """Chunk-local log-gate sums a, li, g (see oracle.c)."""
    ig, fg = _f64(igate_pre), _f64(fgate_pre)
    nc = -(-T // L)
    w = dqk if kind == GLA else 1
    a = np.empty((B, H, T, w), dtype=np.float64)
    li = np.empty((B, H, T), dtype=np.float64)
    g = np.empty((B, H, nc, w), dtype=np.float64)
    rc = _load().oracle_log_gates(_ptr(ig), _ptr(fg), _ptr(a), _ptr(li), _ptr(g),
                                  B, H, T, dqk, L, kind)
    if rc != 0:
        raise ValueError("oracle_log_gates rejected its arguments")
    if kind != GLA:
        a, g = a[..., 0], g[..., 0]
    return a, li, g


# ----------------------------------------------------------------------------
# numpy float64 forms (tiny inputs only)
# ----------------------------------------------------------------------------

def _np_sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def gates_np(igate_pre, fgate_pre, kind, B, H, T, dqk):
    """Per-step gates in float64: i [B,H,T], f [B,H,T,dqk] (channel-constant
    unless kind == GLA)."""
    if kind == MLSTM_SIG:
        i = _np_sigmoid(igate_pre)
        f = np.repeat(_np_sigmoid(fgate_pre)[..., None], dqk, axis=-1)
    elif kind == SCALAR:
        i = np.ones((B, H, T))
        gam = _np_sigmoid(np.asarray(fgate_pre, dtype=np.float64))  # [H]
        f = np.broadcast_to(gam[None, :, None, None], (B, H, T, dqk)).copy()
    elif kind == GLA:
        x = np.asarray(fgate_pre, dtype=np.float64)
        ls = np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))
        i = np.ones((B, H, T))
        f = np.exp(ls / 16.0)
    else:
        raise ValueError(kind)
    return i, f


def closed_form_fwd(q, k, v, igate_pre, fgate_pre, kind):
    """Quadratic closed form by brute force: every decay product is formed
    explicitly as a product of forget gates."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    i, f = gates_np(igate_pre, fgate_pre, kind, B, H, T, dqk)
    h = np.zeros((B, H, T, dhv))
    for b in range(B):
        for hh in range(H):
            for t in range(T):
                acc = np.zeros(dhv)
                for s in range(t + 1):
                    decay = np.prod(f[b, hh, s + 1:t + 1, :], axis=0)  # per channel
                    w = np.sum(q[b, hh, t] * k[b, hh, s] * decay) * i[b, hh, s]
                    acc += w * v[b, hh, s]
                h[b, hh, t] = acc / np.sqrt(dqk)
    return h


def chunkwise_fwd(q, k, v, igate_pre, fgate_pre, kind, L):
    """Chunkwise form: states at chunk boundaries plus masked intra-chunk
    products, all in float64.  Any L >= 1; the last chunk may be partial.
    Returns (h, states after every full chunk [B,H,T//L,dqk,dhv])."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, H, T, dqk = q.shape
    dhv = v.shape[-1]
    i, f = gates_np(igate_pre, fgate_pre, kind, B, H, T, dqk)
    h = np.zeros((B, H, T, dhv))
    states = np.zeros((B, H, T // L, dqk, dhv))
    for b in range(B):
        for hh in range(H):
            C = np.zeros((dqk, dhv))
            for kc, t0 in enumerate(range(0, T, L)):
                t1 = min(t0 + L, T)
                n = t1 - t0
                Q, K, V = q[b, hh, t0:t1], k[b, hh, t0:t1], v[b, hh, t0:t1]
                fc, ic = f[b, hh, t0:t1], i[b, hh, t0:t1]
                # F[t] = prod_{r=t0..t} f_r  (decay from the chunk start)
                F = np.cumprod(fc, axis=0)
                # D[t,s,c] = prod_{r=s+1..t} f_{r,c} for s <= t, 0 above the diagonal
                D = np.zeros((n, n, dqk))
                for s in range(n):
                    D[s, s] = 1.0
                    if s + 1 < n:
                        D[s + 1:, s] = np.cumprod(fc[s + 1:], axis=0)
                W = np.einsum("tc,sc,tsc->ts", Q, K, D) * ic[None, :]
                inter = (Q * F) @ C
                h[b, hh, t0:t1] = (inter + W @ V) / np.sqrt(dqk)
                # state after the chunk: decay to its last step, then add the chunk
                w_s = D[n - 1] * ic[:, None]          # [s, c] = prod_{r=s+1..end} f * i_s
                C = F[n - 1][:, None] * C + (K * w_s).T @ V
                if n == L:
                    states[b, hh, kc] = C
    return h, states

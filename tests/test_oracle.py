"""Pins of the CPU oracle against what the mathematics fixes (no GPU).

The recurrent oracle (plain C, double) is checked against independent
evaluations of the same function: the quadratic closed form by brute force,
causal linear attention (all gates one), the RetNet parallel form (fixed
per-head decay), hand-worked examples, the chunkwise form at every chunk
size, and invariants.  A mistake in the oracle -- a dropped term, a wrong
sign, a shifted time index, a transposed operand -- fails at least one.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import GLA, MLSTM_SIG, SCALAR

REL = 1e-12


def rel_err(x, ref):
    x, ref = np.asarray(x), np.asarray(ref)
    m = np.max(np.abs(ref))
    return np.max(np.abs(x - ref)) / (m if m > 0 else 1.0)


def rand_case(kind, B, H, T, dqk, dhv, seed, gate_scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dqk))
    k = rng.standard_normal((B, H, T, dqk))
    v = rng.standard_normal((B, H, T, dhv))
    if kind == MLSTM_SIG:
        ig = rng.standard_normal((B, H, T)) * 2.0 * gate_scale
        fg = rng.uniform(-2.0, 4.0, (B, H, T)) * gate_scale
    elif kind == SCALAR:
        ig = None
        fg = rng.uniform(-1.0, 5.0, (H,))
    else:
        ig = None
        fg = rng.standard_normal((B, H, T, dqk)) * 3.0 * gate_scale
    return q, k, v, ig, fg


SHAPES = [(2, 2, 1, 1, 1), (2, 2, 2, 3, 4), (2, 2, 7, 8, 1), (2, 2, 33, 3, 8), (2, 2, 48, 8, 4),
          (1, 3, 17, 1, 8)]


@pytest.mark.parametrize("kind", [MLSTM_SIG, SCALAR, GLA])
@pytest.mark.parametrize("shape", SHAPES)
def test_recurrence_equals_closed_form(kind, shape):
    B, H, T, dqk, dhv = shape
    q, k, v, ig, fg = rand_case(kind, B, H, T, dqk, dhv, seed=hash((kind,) + shape) % 2**32)
    h = oracle.recurrent_fwd(q, k, v, ig, fg, kind)
    ref = oracle.closed_form_fwd(q, k, v, ig, fg, kind)
    assert rel_err(h, ref) <= REL


@pytest.mark.parametrize("kind", [MLSTM_SIG, SCALAR, GLA])
def test_unit_gates_give_causal_linear_attention(kind):
    """i = f = 1 reduces the method to causal linear attention:
    h = tril(Q K^T) V / sqrt(d_qk) ("Transformers are RNNs", on the TFLA
    index page's builds-on list)."""
    B, H, T, dqk, dhv = 2, 3, 29, 8, 5
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((B, H, T, d)) for d in (dqk, dqk, dhv))
    if kind == MLSTM_SIG:
        ig, fg = np.full((B, H, T), np.inf), np.full((B, H, T), np.inf)
    elif kind == SCALAR:
        ig, fg = None, np.full((H,), np.inf)
    else:
        ig, fg = None, np.full((B, H, T, dqk), np.inf)
    h = oracle.recurrent_fwd(q, k, v, ig, fg, kind)
    ref = np.tril(q @ np.swapaxes(k, -1, -2)) @ v / math.sqrt(dqk)
    assert rel_err(h, ref) <= REL


def test_scalar_decay_equals_retnet_parallel_form():
    """Fixed decay gamma_h: h = ((Q K^T) * D) V / sqrt(d), D_ts = gamma^(t-s)
    for s <= t (the parallel retention form)."""
    B, H, T, dqk, dhv = 2, 4, 40, 6, 3
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((B, H, T, d)) for d in (dqk, dqk, dhv))
    logits = np.array([math.log(2.0 ** (5 + hh / 4) - 1) for hh in range(H)])
    h = oracle.recurrent_fwd(q, k, v, None, logits, SCALAR)
    gam = 1.0 - 2.0 ** -(5 + np.arange(H) / 4)
    t = np.arange(T)
    expo = t[:, None] - t[None, :]
    D = np.where(expo >= 0, np.power(gam[:, None, None], np.maximum(expo, 0)), 0.0)
    ref = (q @ np.swapaxes(k, -1, -2) * D[None]) @ v / math.sqrt(dqk)
    assert rel_err(h, ref) <= REL


@pytest.mark.parametrize("kind", [MLSTM_SIG, SCALAR, GLA])
@pytest.mark.parametrize("T", [24, 37])
def test_chunkwise_equals_recurrence_for_every_chunk_size(kind, T):
    """The chunkwise form gives the same function for every chunk size; L = 1
    is the recurrence and L >= T the closed form.  Ragged last chunks
    (L not dividing T) included.  The states at chunk ends match too."""
    B, H, dqk, dhv = 1, 2, 4, 3
    q, k, v, ig, fg = rand_case(kind, B, H, T, dqk, dhv, seed=5 + T + kind)
    for L in range(1, T + 2):
        h_rec, st_rec = oracle.recurrent_fwd(q, k, v, ig, fg, kind, L=L)
        h_ch, st_ch = oracle.chunkwise_fwd(q, k, v, ig, fg, kind, L)
        assert rel_err(h_ch, h_rec) <= REL, L
        if st_rec.size:
            assert rel_err(st_ch, st_rec) <= REL, L


def test_hand_worked_scalar_example():
    """d_qk = d_hv = 1, mLSTMsig with pre-activations 0 (i = f = 1/2):
        C1 = 1/2*k1*v1          = 1/2*1*2 = 1      h1 = C1*q1 = 1
        C2 = 1/2*C1 + 1/2*k2*v2 = 1/2 + 1/2 = 1    h2 = C2*q2 = 2
        C3 = 1/2*C2 + 1/2*k3*v3 = 1/2 + 4   = 4.5  h3 = C3*q3 = 4.5
    The first forget gate multiplies C0 = 0 and has no effect."""
    q = np.array([1.0, 2.0, 1.0]).reshape(1, 1, 3, 1)
    k = np.array([1.0, 1.0, 2.0]).reshape(1, 1, 3, 1)
    v = np.array([2.0, 1.0, 4.0]).reshape(1, 1, 3, 1)
    ig = np.zeros((1, 1, 3))
    fg = np.zeros((1, 1, 3))
    h = oracle.recurrent_fwd(q, k, v, ig, fg, MLSTM_SIG)
    assert np.array_equal(h.ravel(), [1.0, 2.0, 4.5])


def test_hand_worked_matrix_example():
    """d_qk = 2, d_hv = 3, i = 1 (pre-activation +inf), f = 1/2:
        C1 = k1 v1^T = [[1,2,3],[2,4,6]]             h1 = C1^T q1 / sqrt2 = (2,4,6)/sqrt2
        C2 = C1/2 + k2 v2^T = [[1/2,2,3/2],[1,2,3]]  h2 = C2^T q2 / sqrt2 = (1/2,2,3/2)/sqrt2
    with q1 = (0,1), k1 = (1,2), v1 = (1,2,3), q2 = (1,0), k2 = (1,0), v2 = (0,1,0).
    A transposed state or a swapped q/k would give different numbers."""
    q = np.array([[0.0, 1.0], [1.0, 0.0]]).reshape(1, 1, 2, 2)
    k = np.array([[1.0, 2.0], [1.0, 0.0]]).reshape(1, 1, 2, 2)
    v = np.array([[1.0, 2.0, 3.0], [0.0, 1.0, 0.0]]).reshape(1, 1, 2, 3)
    ig = np.full((1, 1, 2), np.inf)
    fg = np.zeros((1, 1, 2))
    h = oracle.recurrent_fwd(q, k, v, ig, fg, MLSTM_SIG)
    r2 = math.sqrt(2.0)
    expect = np.array([[2.0, 4.0, 6.0], [0.5, 2.0, 1.5]]) / r2
    assert np.allclose(h[0, 0], expect, rtol=0, atol=1e-15)


@pytest.mark.parametrize("kind", [MLSTM_SIG, GLA])
def test_single_step(kind):
    """T = 1: h1 = i1 (q1 . k1) v1 / sqrt(d) whatever the forget gate."""
    q, k, v, ig, fg = rand_case(kind, 2, 2, 1, 5, 3, seed=3)
    h = oracle.recurrent_fwd(q, k, v, ig, fg, kind)
    i = 1.0 / (1.0 + np.exp(-ig)) if kind == MLSTM_SIG else np.ones((2, 2, 1))
    ref = i[..., None] * np.sum(q * k, axis=-1, keepdims=True) * v / math.sqrt(5)
    assert rel_err(h, ref) <= REL


def test_zero_forget_gate_forgets_everything():
    """f = 0 (pre-activation -inf) everywhere: h_t = i_t (q_t . k_t) v_t / sqrt(d)."""
    q, k, v, ig, _ = rand_case(MLSTM_SIG, 2, 2, 9, 4, 3, seed=4)
    fg = np.full((2, 2, 9), -np.inf)
    h = oracle.recurrent_fwd(q, k, v, ig, fg, MLSTM_SIG)
    i = 1.0 / (1.0 + np.exp(-ig))
    ref = i[..., None] * np.sum(q * k, axis=-1, keepdims=True) * v / math.sqrt(4)
    assert rel_err(h, ref) <= REL
    # the same through a per-channel gate
    x = np.full((2, 2, 9, 4), -np.inf)
    h2 = oracle.recurrent_fwd(q, k, v, None, x, GLA)
    ref2 = np.sum(q * k, axis=-1, keepdims=True) * v / math.sqrt(4)
    assert rel_err(h2, ref2) <= REL


def test_zero_input_gate_gives_zero():
    q, k, v, _, fg = rand_case(MLSTM_SIG, 1, 2, 8, 3, 3, seed=9)
    ig = np.full((1, 2, 8), -np.inf)
    h = oracle.recurrent_fwd(q, k, v, ig, fg, MLSTM_SIG)
    assert np.all(h == 0.0)


@pytest.mark.parametrize("kind", [MLSTM_SIG, SCALAR, GLA])
def test_invariants(kind):
    B, H, T, dqk, dhv = 2, 3, 21, 4, 5
    q, k, v, ig, fg = rand_case(kind, B, H, T, dqk, dhv, seed=21 + kind)
    h = oracle.recurrent_fwd(q, k, v, ig, fg, kind)
    # the first forget gate multiplies C0 = 0
    if kind != SCALAR:
        fg2 = fg.copy()
        fg2[:, :, 0] = -fg2[:, :, 0] + 1.3
        assert np.array_equal(oracle.recurrent_fwd(q, k, v, ig, fg2, kind), h)
    # causality: changing step >= t0 leaves h_{<t0} bit-identical
    t0 = 11
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, :, t0:] += 1.0
    k2[:, :, t0:] -= 2.0
    v2[:, :, t0:] *= 3.0
    h2 = oracle.recurrent_fwd(q2, k2, v2, ig, fg, kind)
    assert np.array_equal(h2[:, :, :t0], h[:, :, :t0])
    assert not np.array_equal(h2[:, :, t0:], h[:, :, t0:])
    # linear in v, homogeneous of degree one in q and in k
    v3 = np.random.default_rng(1).standard_normal(v.shape)
    hv = oracle.recurrent_fwd(q, k, v + 2.5 * v3, ig, fg, kind)
    hv3 = oracle.recurrent_fwd(q, k, v3, ig, fg, kind)
    assert rel_err(hv, h + 2.5 * hv3) <= REL
    assert rel_err(oracle.recurrent_fwd(-3.0 * q, k, v, ig, fg, kind), -3.0 * h) <= REL
    assert rel_err(oracle.recurrent_fwd(q, 0.5 * k, v, ig, fg, kind), 0.5 * h) <= REL
    # heads are independent: permuting (b, h) permutes outputs
    if kind != SCALAR:
        perm = np.random.default_rng(2).permutation(B * H)

        def p(a):
            if a is None:
                return None
            s = a.shape
            return a.reshape((B * H,) + s[2:])[perm].reshape(s)

        hp = oracle.recurrent_fwd(p(q), p(k), p(v), p(ig), p(fg), kind)
        assert np.array_equal(hp, p(h))


def test_channel_constant_gla_equals_scalar_gate_core():
    """A per-channel gate that is the same on every channel is a per-step
    scalar gate: GLA with x[t, c] = x[t] equals mLSTMsig with i = 1 and
    f = exp(logsigmoid(x)/16)."""
    B, H, T, dqk, dhv = 1, 2, 19, 4, 3
    rng = np.random.default_rng(33)
    q, k, v = (rng.standard_normal((B, H, T, d)) for d in (dqk, dqk, dhv))
    x = rng.standard_normal((B, H, T)) * 2.0
    h_gla = oracle.recurrent_fwd(q, k, v, None, np.repeat(x[..., None], dqk, axis=-1), GLA)
    f = np.exp((np.minimum(x, 0) - np.log1p(np.exp(-np.abs(x)))) / 16.0)
    fpre = np.log(f) - np.log1p(-f)           # logit(f)
    h_sig = oracle.recurrent_fwd(q, k, v, np.full((B, H, T), np.inf), fpre, MLSTM_SIG)
    assert rel_err(h_sig, h_gla) <= 1e-11


def test_gate_functions():
    for x in [-30.0, -5.0, -0.5, 0.0, 0.25, 3.0, 17.0]:
        assert oracle.log_sigmoid(x) == pytest.approx(-math.log1p(math.exp(-x)), rel=1e-14, abs=1e-300)
        assert oracle.sigmoid(x) == pytest.approx(1.0 / (1.0 + math.exp(-x)), rel=1e-14)
    for x in [-80.0, 80.0, -700.0, 700.0]:
        assert math.isfinite(oracle.log_sigmoid(x))
    assert oracle.log_sigmoid(-80.0) == pytest.approx(-80.0, rel=1e-15)
    assert oracle.sigmoid(math.inf) == 1.0 and oracle.sigmoid(-math.inf) == 0.0
    assert oracle.log_sigmoid(math.inf) == 0.0 and oracle.log_sigmoid(-math.inf) == -math.inf


@pytest.mark.parametrize("kind", [MLSTM_SIG, SCALAR, GLA])
def test_log_gate_sums_are_log_decay_products(kind):
    """exp(a_t - a_s) is the product of the forget gates strictly after s up
    to t inside a chunk, exp(a_t) the product from the chunk start, exp(li)
    the input gate, g the value at the chunk's last step."""
    B, H, T, dqk, L = 1, 2, 23, 3, 8
    q, k, v, ig, fg = rand_case(kind, B, H, T, dqk, 2, seed=44 + kind)
    a, li, g = oracle.log_gates(ig, fg, kind, B, H, T, dqk, L)
    i, f = oracle.gates_np(ig, fg, kind, B, H, T, dqk)
    if kind != GLA:
        a, g = a[..., None], g[..., None]
    for t0 in range(0, T, L):
        t1 = min(t0 + L, T)
        for t in range(t0, t1):
            assert np.allclose(np.exp(a[:, :, t]), np.prod(f[:, :, t0:t + 1], axis=2)[..., :a.shape[-1]],
                               rtol=1e-12, atol=0)
        assert np.array_equal(g[:, :, t0 // L], a[:, :, t1 - 1])
    assert np.allclose(np.exp(li), i, rtol=1e-13, atol=0)


@pytest.mark.parametrize("kind", [MLSTM_SIG, SCALAR, GLA])
def test_initial_state_splits_a_sequence(kind):
    """Running steps [0, t1) and then [t1, T) from the first part's final
    state reproduces the whole sequence: outputs and final state."""
    B, H, T, dqk, dhv = 2, 2, 31, 5, 4
    q, k, v, ig, fg = rand_case(kind, B, H, T, dqk, dhv, seed=70 + kind)
    h_all, c_all = oracle.recurrent_fwd_state(q, k, v, ig, fg, kind)
    for t1 in (1, 13, 30):
        def part(a, lo, hi):
            if a is None or kind == SCALAR and a is fg:
                return a
            return a[:, :, lo:hi]
        h1, c1 = oracle.recurrent_fwd_state(part(q, 0, t1), part(k, 0, t1), part(v, 0, t1), part(ig, 0, t1),
                                            part(fg, 0, t1), kind)
        h2, c2 = oracle.recurrent_fwd_state(part(q, t1, T), part(k, t1, T), part(v, t1, T), part(ig, t1, T),
                                            part(fg, t1, T), kind, c0=c1)
        assert rel_err(np.concatenate([h1, h2], axis=2), h_all) <= REL
        assert rel_err(c2, c_all) <= REL


def test_initial_state_closed_form():
    """With an initial state, h_t gains (prod_{r<=t} f_r) C_0^T q_t / sqrt(d)
    on top of the zero-start result; the final state gains prod_{r<=T} f_r C_0."""
    B, H, T, dqk, dhv = 1, 2, 17, 4, 3
    q, k, v, ig, fg = rand_case(MLSTM_SIG, B, H, T, dqk, dhv, seed=81)
    c0 = np.random.default_rng(82).standard_normal((B, H, dqk, dhv))
    h0, cT0 = oracle.recurrent_fwd_state(q, k, v, ig, fg, MLSTM_SIG)
    h1, cT1 = oracle.recurrent_fwd_state(q, k, v, ig, fg, MLSTM_SIG, c0=c0)
    f = 1.0 / (1.0 + np.exp(-fg))                       # [B,H,T]
    F = np.cumprod(f, axis=2)
    extra = F[..., None] * np.einsum("bhtc,bhcj->bhtj", q, c0) / math.sqrt(dqk)
    assert rel_err(h1, h0 + extra) <= REL
    assert rel_err(cT1, cT0 + F[:, :, -1, None, None] * c0) <= REL


# ---------------------------------------------------------------- backward pass
def _all_inputs(kind, B, H, T, dqk, dhv, seed):
    q, k, v, ig, fg = rand_case(kind, B, H, T, dqk, dhv, seed=seed)
    dh = np.random.default_rng(seed + 1).standard_normal((B, H, T, dhv))
    return q, k, v, ig, fg, dh


@pytest.mark.parametrize("kind", [MLSTM_SIG, SCALAR, GLA])
def test_backward_matches_finite_differences(kind):
    """Every gradient of L = sum(dh * h) against central differences of the
    forward recurrence, element by element."""
    B, H, T, dqk, dhv = 1, 2, 6, 3, 2
    q, k, v, ig, fg, dh = _all_inputs(kind, B, H, T, dqk, dhv, seed=40 + kind)
    grads = oracle.recurrent_bwd(q, k, v, ig, fg, dh, kind)
    names = ["q", "k", "v", "ig", "fg"]
    arrs = {"q": q, "k": k, "v": v, "ig": ig, "fg": fg}

    def loss(a):
        return float(np.sum(dh * oracle.recurrent_fwd(a["q"], a["k"], a["v"], a["ig"], a["fg"], kind)))

    eps = 1e-6
    for name, g in zip(names, [grads[0], grads[1], grads[2], grads[3], grads[4]]):
        if arrs[name] is None:
            assert g is None
            continue
        num = np.empty_like(arrs[name])
        for idx in np.ndindex(arrs[name].shape):
            plus = {n: (a.copy() if a is not None else None) for n, a in arrs.items()}
            minus = {n: (a.copy() if a is not None else None) for n, a in arrs.items()}
            plus[name][idx] += eps
            minus[name][idx] -= eps
            num[idx] = (loss(plus) - loss(minus)) / (2 * eps)
        assert rel_err(g, num) <= 1e-6, name


def _closed_form_torch(q, k, v, ig, fg, kind):
    """The quadratic closed form in float64 torch ops (cumulative log forget
    gates, explicit decay matrix), differentiated by autograd."""
    import torch
    B, H, T, dqk = q.shape
    if kind == MLSTM_SIG:
        lf = torch.nn.functional.logsigmoid(fg)                                  # [B,H,T]
        li = torch.nn.functional.logsigmoid(ig)
        cum = torch.cumsum(lf, dim=-1)
        logd = cum[..., :, None] - cum[..., None, :] + li[..., None, :]          # [B,H,t,s]
        s = q @ k.transpose(-1, -2)
    elif kind == SCALAR:
        lf = torch.nn.functional.logsigmoid(fg)                                  # [H]
        t = torch.arange(T, dtype=torch.float64)
        logd = (t[:, None] - t[None, :])[None, None] * lf[None, :, None, None]
        s = q @ k.transpose(-1, -2)
    else:
        lf = torch.nn.functional.logsigmoid(fg) / 16.0                           # [B,H,T,c]
        cum = torch.cumsum(lf, dim=2)
        # per channel decay inside q.k; mask before exponentiating (no inf * 0)
        diff = cum[:, :, :, None, :] - cum[:, :, None, :, :]                     # [B,H,t,s,c]
        mask = torch.tril(torch.ones(T, T, dtype=torch.bool))[None, None, :, :, None]
        diff = torch.where(mask, diff, torch.full_like(diff, -1e9))
        s = torch.einsum("bhtc,bhsc,bhtsc->bhts", q, k, torch.exp(diff))
        logd = torch.zeros_like(s)
    causal = torch.tril(torch.ones(T, T, dtype=torch.bool))
    logd = torch.where(causal, logd, torch.full_like(logd, -1e9))
    return (s * torch.exp(logd)) @ v / math.sqrt(dqk)


@pytest.mark.parametrize("kind", [MLSTM_SIG, SCALAR, GLA])
def test_backward_matches_autograd_of_closed_form(kind):
    import torch
    B, H, T, dqk, dhv = 2, 2, 21, 4, 5
    q, k, v, ig, fg, dh = _all_inputs(kind, B, H, T, dqk, dhv, seed=50 + kind)
    tt = {n: (None if a is None else torch.tensor(a, dtype=torch.float64, requires_grad=True))
          for n, a in zip(["q", "k", "v", "ig", "fg"], [q, k, v, ig, fg])}
    h = _closed_form_torch(tt["q"], tt["k"], tt["v"], tt["ig"], tt["fg"], kind)
    (h * torch.tensor(dh)).sum().backward()
    got = oracle.recurrent_bwd(q, k, v, ig, fg, dh, kind)
    for name, g in zip(["q", "k", "v", "ig", "fg"], got):
        if tt[name] is None:
            continue
        assert rel_err(g, tt[name].grad.numpy()) <= 1e-10, name


def _forget_grad_by_pairs(q, k, v, ig, fg, dh, kind):
    """dL/dfgate_pre by brute force over the step pairs a forget gate couples.
    h_t = sum_{s<=t} D_ts i_s (q_t . k_s) v_s / sqrt(d) with
    D_ts = prod_{r=s+1..t} f_r, so dD_ts/dlog f_j = D_ts exactly when
    s < j <= t: dL/dlog f_j = sum_{t>=j} sum_{s<j} D_ts i_s (q_t . k_s)
    (dh_t . v_s) / sqrt(d) (per key channel c for the per-channel gate,
    with q_t,c k_s,c in place of q_t . k_s).  Every term is formed as a
    product of positive decays, so gradients of size e^-250 keep their
    relative precision.  Then through the gate functions."""
    B, H, T, dqk = q.shape
    sig = lambda x: 0.5 * (1.0 + np.tanh(0.5 * x))                 # no overflow at |x| = 2000
    logsig = lambda x: np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))
    out = np.zeros(fg.shape)
    for b in range(B):
        for hd in range(H):
            if kind == MLSTM_SIG:
                lf = logsig(fg[b, hd])[:, None] * np.ones((1, dqk))
                i = sig(ig[b, hd])
            elif kind == SCALAR:
                lf = np.full((T, dqk), logsig(fg[hd]))
                i = np.ones(T)
            else:
                lf = logsig(fg[b, hd]) / 16.0
                i = np.ones(T)
            g = np.zeros((T, dqk))
            for j in range(T):
                for t in range(j, T):
                    for s_ in range(j):
                        D = np.exp(np.sum(lf[s_ + 1:t + 1], axis=0))          # [dqk]
                        g[j] += D * i[s_] * q[b, hd, t] * k[b, hd, s_] * np.dot(dh[b, hd, t], v[b, hd, s_])
            g /= math.sqrt(dqk)
            if kind == MLSTM_SIG:
                out[b, hd] = g.sum(axis=1) * sig(-fg[b, hd])
            elif kind == SCALAR:
                out[hd] += g.sum() * sig(-fg[hd])
            else:
                out[b, hd] = g * sig(-fg[b, hd]) / 16.0
    return out


@pytest.mark.parametrize("kind", [MLSTM_SIG, SCALAR, GLA])
def test_backward_is_the_plain_derivative_for_vanishing_forget_gates(kind):
    """Forget gates far below e^-100 (a log forget gate of -250, or -125 per
    key channel): the gradient of their pre-activation is the plain
    derivative -- tiny but not zero -- element by element against the
    brute-force pair sum (a floor on the log gate would zero exactly these
    entries); the other gradients against float64 autograd of the
    quadratic closed form."""
    import torch
    B, H, T, dqk, dhv = 1, 2, 9, 3, 4
    q, k, v, ig, fg, dh = _all_inputs(kind, B, H, T, dqk, dhv, seed=55 + kind)
    if kind == MLSTM_SIG:
        fg[0, 0, [2, 5]] = -250.0
        extreme = np.zeros(fg.shape, bool)
        extreme[0, 0, [2, 5]] = True
    elif kind == SCALAR:
        fg[1] = -250.0
        extreme = np.array([False, True])
    else:
        fg[0, 1, 4, :2] = -2000.0          # log f = logsigmoid(-2000) / 16 = -125
        extreme = np.zeros(fg.shape, bool)
        extreme[0, 1, 4, :2] = True
    got = oracle.recurrent_bwd(q, k, v, ig, fg, dh, kind)
    ref = _forget_grad_by_pairs(q, k, v, ig, fg, dh, kind)
    assert rel_err(got[4], ref) <= 1e-10
    assert np.all(ref[extreme] != 0.0) and np.all(np.abs(ref[extreme]) < 1e-50)
    np.testing.assert_allclose(got[4][extreme], ref[extreme], rtol=1e-9, atol=0.0)
    tt = {n: (None if a is None else torch.tensor(a, dtype=torch.float64, requires_grad=True))
          for n, a in zip(["q", "k", "v", "ig"], [q, k, v, ig])}
    h = _closed_form_torch(tt["q"], tt["k"], tt["v"], tt["ig"], torch.tensor(fg), kind)
    (h * torch.tensor(dh)).sum().backward()
    for name, g in zip(["q", "k", "v", "ig"], got):
        if tt[name] is not None:
            assert rel_err(g, tt[name].grad.numpy()) <= 1e-10, name


def test_backward_of_a_zero_forget_gate():
    """f = sigmoid(-inf) = 0: dh/dfgate_pre = f (1 - f) dL/df = 0 at that
    step exactly, and the other gradients are finite and match the reverse
    sum identity dL/dlog f_t = sum_{t' >= t} (q.dq - k.dk) times (1 - f)."""
    B, H, T, dqk, dhv = 1, 1, 12, 3, 2
    q, k, v, ig, fg, dh = _all_inputs(MLSTM_SIG, B, H, T, dqk, dhv, seed=57)
    fg[0, 0, 6] = -np.inf
    dq, dk, dv, dig, dfg = oracle.recurrent_bwd(q, k, v, ig, fg, dh, MLSTM_SIG)
    assert dfg[0, 0, 6] == 0.0
    for g in (dq, dk, dv, dig, dfg):
        assert np.all(np.isfinite(g))
    r = np.sum(q * dq - k * dk, axis=-1)
    dlogf = np.flip(np.cumsum(np.flip(r, -1), -1), -1)
    f = 1.0 / (1.0 + np.exp(-fg))
    assert rel_err(dlogf * (1.0 - f), dfg) <= 1e-10


@pytest.mark.parametrize("kind", [MLSTM_SIG, GLA])
def test_forget_gradient_is_reverse_sum_of_q_dq_minus_k_dk(kind):
    """dL/dlog f_t = sum over t' >= t of (q_t' . dq_t' - k_t' . dk_t'),
    per key channel for the per-channel gate (the form the GPU backward
    evaluates), against the oracle's direct df."""
    B, H, T, dqk, dhv = 2, 1, 40, 6, 3
    q, k, v, ig, fg, dh = _all_inputs(kind, B, H, T, dqk, dhv, seed=60 + kind)
    dq, dk, dv, dig, dfg = oracle.recurrent_bwd(q, k, v, ig, fg, dh, kind)
    if kind == MLSTM_SIG:
        r = np.sum(q * dq - k * dk, axis=-1)                      # [B,H,T]
        dlogf = np.flip(np.cumsum(np.flip(r, -1), -1), -1)
        f = 1.0 / (1.0 + np.exp(-fg))
        assert rel_err(dlogf * (1.0 - f), dfg) <= 1e-10
        i = 1.0 / (1.0 + np.exp(-ig))
        assert rel_err(np.sum(k * dk, axis=-1) * (1.0 - i), dig) <= 1e-10
    else:
        r = q * dq - k * dk                                        # [B,H,T,c]
        dlogf = np.flip(np.cumsum(np.flip(r, 2), 2), 2)
        sx = 1.0 / (1.0 + np.exp(-fg))
        assert rel_err(dlogf * (1.0 - sx) / 16.0, dfg) <= 1e-10


# ------------------------------------------------ backward with state in and out
@pytest.mark.parametrize("kind", [MLSTM_SIG, SCALAR, GLA])
def test_state_backward_matches_finite_differences(kind):
    """L = sum(dh * h) + sum(dcT * C_T) from the initial state c0: every
    gradient, dL/dc0 included, against central differences of the forward
    recurrence from that state."""
    B, H, T, dqk, dhv = 1, 2, 5, 3, 2
    q, k, v, ig, fg, dh = _all_inputs(kind, B, H, T, dqk, dhv, seed=70 + kind)
    rng = np.random.default_rng(80 + kind)
    c0 = rng.standard_normal((B, H, dqk, dhv))
    dcT = rng.standard_normal((B, H, dqk, dhv))
    got = oracle.recurrent_bwd_state(q, k, v, ig, fg, dh, kind, c0=c0, dcT=dcT)
    arrs = {"q": q, "k": k, "v": v, "ig": ig, "fg": fg, "c0": c0}

    def loss(a):
        h, cT = oracle.recurrent_fwd_state(a["q"], a["k"], a["v"], a["ig"], a["fg"], kind, c0=a["c0"])
        return float(np.sum(dh * h) + np.sum(dcT * cT))

    eps = 1e-6
    for name, g in zip(["q", "k", "v", "ig", "fg", "c0"], got):
        if arrs[name] is None:
            assert g is None
            continue
        num = np.empty_like(arrs[name])
        for idx in np.ndindex(arrs[name].shape):
            plus = {n: (x.copy() if x is not None else None) for n, x in arrs.items()}
            minus = {n: (x.copy() if x is not None else None) for n, x in arrs.items()}
            plus[name][idx] += eps
            minus[name][idx] -= eps
            num[idx] = (loss(plus) - loss(minus)) / (2 * eps)
        assert rel_err(g, num) <= 1e-6, name


@pytest.mark.parametrize("kind", [MLSTM_SIG, GLA])
def test_state_backward_chains_over_a_split_sequence(kind):
    """The backward of a sequence equals that of its two halves chained: the
    second half starts from the first half's final state, and its dL/dC_0 is
    the first half's final-state gradient."""
    B, H, T, dqk, dhv = 2, 1, 37, 4, 3
    q, k, v, ig, fg, dh = _all_inputs(kind, B, H, T, dqk, dhv, seed=90 + kind)
    whole = oracle.recurrent_bwd(q, k, v, ig, fg, dh, kind)
    m = 16
    cut = lambda x, a, b: None if x is None else x[:, :, a:b]
    _, c_mid = oracle.recurrent_fwd_state(cut(q, 0, m), cut(k, 0, m), cut(v, 0, m), cut(ig, 0, m), cut(fg, 0, m), kind)
    second = oracle.recurrent_bwd_state(cut(q, m, T), cut(k, m, T), cut(v, m, T), cut(ig, m, T), cut(fg, m, T),
                                        cut(dh, m, T), kind, c0=c_mid)
    first = oracle.recurrent_bwd_state(cut(q, 0, m), cut(k, 0, m), cut(v, 0, m), cut(ig, 0, m), cut(fg, 0, m),
                                       cut(dh, 0, m), kind, dcT=second[5])
    for i in range(5):
        if whole[i] is None:
            continue
        joined = np.concatenate([first[i], second[i]], axis=2)
        assert rel_err(joined, whole[i]) <= 1e-12, i
    assert np.abs(first[5]).max() > 0      # a gradient reaches the zero initial state


def test_state_backward_without_states_is_the_plain_backward():
    q, k, v, ig, fg, dh = _all_inputs(MLSTM_SIG, 1, 2, 30, 4, 5, seed=99)
    a = oracle.recurrent_bwd(q, k, v, ig, fg, dh, MLSTM_SIG)
    b = oracle.recurrent_bwd_state(q, k, v, ig, fg, dh, MLSTM_SIG)
    for x, y in zip(a, b[:5]):
        assert np.array_equal(x, y)

"""Pins of the mLSTMexp oracle (exponential input gate, normaliser state,
max state; no GPU).

The pages name mLSTMexp only in words (TFLA research-map summary, Approach:
the exponential input gate with normaliser and max state that mLSTMsig
replaces); no value for it is printed.  The recurrent oracle with its max
state is pinned here against what the mathematics fixes: the plain
definition by brute force, the chunkwise form at every chunk size, the
invariance of h under a shift of every input-gate pre-activation once the
normaliser is active (which the max state must preserve far past the range
where exp overflows), the reduction to the normaliser-free recurrence when
the normaliser never reaches 1, a single step, vanishing gates, a
hand-worked example and causality.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import MLSTM_SIG


def rel_err(x, ref):
    m = np.max(np.abs(ref))
    return np.max(np.abs(np.asarray(x) - ref)) / (m if m > 0 else 1.0)


def case(B, H, T, dqk, dhv, seed, ig_mean=0.0, ig_std=2.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dqk))
    k = rng.standard_normal((B, H, T, dqk))
    v = rng.standard_normal((B, H, T, dhv))
    ig = ig_mean + ig_std * rng.standard_normal((B, H, T))
    fg = rng.uniform(-2.0, 4.0, (B, H, T))
    return q, k, v, ig, fg


def denominators(q, k, ig, fg):
    """|den_t| of the plain definition, brute force (the normaliser term)."""
    B, H, T, dqk = q.shape
    f = 1.0 / (1.0 + np.exp(-fg))
    out = np.zeros((B, H, T))
    for b in range(B):
        for hd in range(H):
            for t in range(T):
                den = sum(np.prod(f[b, hd, s + 1:t + 1]) * math.exp(ig[b, hd, s]) * np.dot(q[b, hd, t], k[b, hd, s])
                          for s in range(t + 1))
                out[b, hd, t] = abs(den) / math.sqrt(dqk)
    return out


@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1), (2, 2, 2, 3, 4), (2, 2, 7, 8, 1), (2, 2, 33, 3, 8),
                                   (1, 3, 40, 8, 4)])
def test_exp_recurrence_equals_plain_definition(shape):
    q, k, v, ig, fg = case(*shape, seed=sum(shape))
    h = oracle.recurrent_fwd_exp(q, k, v, ig, fg)
    assert rel_err(h, oracle.closed_form_fwd_exp(q, k, v, ig, fg)) <= 1e-12


@pytest.mark.parametrize("T", [24, 37])
def test_exp_chunkwise_equals_recurrence_for_every_chunk_size(T):
    q, k, v, ig, fg = case(2, 2, T, 4, 3, seed=T)
    h = oracle.recurrent_fwd_exp(q, k, v, ig, fg)
    for L in range(1, T + 2):
        assert rel_err(oracle.chunkwise_fwd_exp(q, k, v, ig, fg, L), h) <= 1e-12, L


def test_exp_max_state_keeps_h_far_past_overflow():
    """Once |den_t| >= 1 at every step, h is invariant under igate_pre + c
    (numerator and denominator scale by e^c).  At c = 800 e^{igate_pre}
    overflows double and the plain definition gives inf/inf; the oracle's
    max state must still give the value of the plain definition at c = 40."""
    q, k, v, ig, fg = case(2, 2, 30, 4, 3, seed=11, ig_std=1.0)
    base = ig + 40.0
    assert np.min(denominators(q, k, base, fg)) >= 1.0
    ref = oracle.closed_form_fwd_exp(q, k, v, base, fg)
    with np.errstate(over="ignore", invalid="ignore"):
        assert not np.all(np.isfinite(oracle.closed_form_fwd_exp(q, k, v, ig + 800.0, fg)))
    for c in (40.0, 300.0, 800.0):
        h = oracle.recurrent_fwd_exp(q, k, v, ig + c, fg)
        assert np.all(np.isfinite(h))
        assert rel_err(h, ref) <= 1e-10, c


def test_exp_without_active_normaliser_is_the_plain_recurrence():
    """With every |den_t| < 1 the normaliser is inactive and h is the
    normaliser-free recurrence with input gate e^{igate_pre}: the mLSTMsig
    oracle given the input-gate pre-activation logit(e^{igate_pre})."""
    q, k, v, ig, fg = case(2, 2, 30, 4, 3, seed=12, ig_mean=-30.0, ig_std=1.0)
    assert np.max(denominators(q, k, ig, fg)) < 1.0
    logit = ig - np.log1p(-np.exp(ig))
    ref = oracle.recurrent_fwd(q, k, v, logit, fg, MLSTM_SIG)
    assert rel_err(oracle.recurrent_fwd_exp(q, k, v, ig, fg), ref) <= 1e-10


def test_exp_single_step():
    """T = 1: h_1 = e^{i} (q.k) v / sqrt(d) / max(e^{i} |q.k| / sqrt(d), 1),
    i.e. v sign(q.k) once the normaliser is active."""
    rng = np.random.default_rng(13)
    q, k = rng.standard_normal((2, 1, 1, 1, 5))
    v = rng.standard_normal((1, 1, 1, 3))
    fg = np.zeros((1, 1, 1))
    qk = float(np.dot(q[0, 0, 0], k[0, 0, 0]))
    for i in (-6.0, 0.0, 8.0):
        ig = np.full((1, 1, 1), i)
        w = math.exp(i) * qk / math.sqrt(5)
        ref = w * v[0, 0, 0] / max(abs(w), 1.0)
        assert rel_err(oracle.recurrent_fwd_exp(q, k, v, ig, fg)[0, 0, 0], ref) <= 1e-13
    ig = np.full((1, 1, 1), 8.0)
    assert rel_err(oracle.recurrent_fwd_exp(q, k, v, ig, fg)[0, 0, 0], np.sign(qk) * v[0, 0, 0]) <= 1e-13


def test_exp_hand_worked_example():
    """d_qk = d_hv = 1 (scale 1), k = 1, v = 3, igate_pre = 0 (i = 1), forget
    gate of step 2 sigmoid(0) = 1/2:
      C_1 = 3, n_1 = 1;  C_2 = 3/2 + 3 = 9/2, n_2 = 1/2 + 1 = 3/2.
    q = 2:    h = (6 / max(2, 1), 9 / max(3, 1))       = (3, 3)
    q = 1/4:  h = (3/4 / max(1/4, 1), 9/8 / max(3/8, 1)) = (3/4, 9/8)."""
    k = np.ones((1, 1, 2, 1))
    v = np.full((1, 1, 2, 1), 3.0)
    ig = np.zeros((1, 1, 2))
    fg = np.array([[[5.0, 0.0]]])
    for qv, ref in ((2.0, [3.0, 3.0]), (0.25, [0.75, 1.125])):
        q = np.full((1, 1, 2, 1), qv)
        h = oracle.recurrent_fwd_exp(q, k, v, ig, fg)
        assert np.allclose(h[0, 0, :, 0], ref, rtol=1e-14, atol=0)


def test_exp_vanishing_gates():
    """Input gates of 0 (igate_pre = -inf) before the first input: h = 0
    there, and the rest equals the run started at the first input; a forget
    gate of 0 at step t erases everything before t."""
    q, k, v, ig, fg = case(1, 2, 25, 4, 3, seed=14)
    ig[:, :, :5] = -np.inf
    h = oracle.recurrent_fwd_exp(q, k, v, ig, fg)
    assert np.all(h[:, :, :5] == 0.0)
    tail = oracle.recurrent_fwd_exp(q[:, :, 5:], k[:, :, 5:], v[:, :, 5:], ig[:, :, 5:], fg[:, :, 5:])
    assert rel_err(h[:, :, 5:], tail) <= 1e-13
    q, k, v, ig, fg = case(1, 2, 25, 4, 3, seed=15)
    fg[:, :, 12] = -np.inf
    h = oracle.recurrent_fwd_exp(q, k, v, ig, fg)
    tail = oracle.recurrent_fwd_exp(q[:, :, 12:], k[:, :, 12:], v[:, :, 12:], ig[:, :, 12:], fg[:, :, 12:])
    assert rel_err(h[:, :, 12:], tail) <= 1e-13


def test_exp_causality_and_value_homogeneity():
    q, k, v, ig, fg = case(2, 1, 20, 4, 3, seed=16)
    h = oracle.recurrent_fwd_exp(q, k, v, ig, fg)
    q2, k2, v2, ig2, fg2 = (x.copy() for x in (q, k, v, ig, fg))
    for x in (q2, k2, v2):
        x[:, :, 12:] += 1.0
    ig2[:, :, 12:] += 3.0
    fg2[:, :, 12:] -= 1.0
    h2 = oracle.recurrent_fwd_exp(q2, k2, v2, ig2, fg2)
    assert np.array_equal(h[:, :, :12], h2[:, :, :12])
    assert rel_err(oracle.recurrent_fwd_exp(q, k, 2.5 * v, ig, fg), 2.5 * h) <= 1e-14

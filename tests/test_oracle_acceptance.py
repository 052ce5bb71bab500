"""Pins of the oracle's direct-sparse-sampling pieces: the drafter's own draws
(draw_tokens) and the acceptance rate alpha = sum_x min(p, q).

* the acceptance rate against its closed forms: q = p gives 1, disjoint
  supports give 0, two tokens give 1 - |p(0) - q(0)| with p(0) a logistic;
* against the total-variation identity alpha = 1 - (1/2) sum_x |p(x) - q(x)|;
* against the speculative sampler itself: the exact vocab-8 enumeration of
  oracle.spec_sample gives P(n >= 1) = alpha_0 and P(n >= 2) = alpha_0 alpha_1;
* the draws against the definition with an independent generator: the uniform
  of coordinate (offset, b, first_slot + r, stream 2) from numpy.random.Philox,
  located in the row's cumulative distribution by numpy.searchsorted.
"""
import math

import numpy as np
import pytest

import oracle
from tests.test_oracle_philox import _numpy_block
from tests.test_oracle_sample import _enumerate


def _probs(logits, T):
    z = np.asarray(logits, dtype=np.float64) / T
    e = np.exp(z - np.max(z))
    return e / e.sum()


def test_acceptance_q_equals_p_is_one():
    rng = np.random.default_rng(0)
    d = rng.normal(0, 2.0, (3, 4, 500))
    t = np.concatenate([d, rng.normal(0, 2.0, (3, 1, 500))], axis=1)
    a = oracle.acceptance_rate(d, t, 0.8)
    assert a.shape == (3, 4)
    np.testing.assert_allclose(a, 1.0, rtol=0, atol=1e-12)


def test_acceptance_disjoint_supports_is_zero():
    rng = np.random.default_rng(1)
    d = rng.normal(0, 1.0, (2, 3, 16))
    t = rng.normal(0, 1.0, (2, 4, 16))
    d[..., :8] = -np.inf   # the drafter only proposes tokens 8..15
    t[:, :3, 8:] = -np.inf  # the target only allows tokens 0..7
    assert np.all(oracle.acceptance_rate(d, t, 1.0) == 0.0)


@pytest.mark.parametrize("a,b,T", [(0.0, 0.0, 1.0), (1.5, -0.5, 1.0), (3.0, 2.0, 0.5), (-4.0, 6.0, 2.0)])
def test_acceptance_two_tokens_closed_form(a, b, T):
    # logits (0, a) and (0, b): p(0) = 1 / (1 + e^(a/T)), q(0) = 1 / (1 + e^(b/T))
    d = np.array([[[0.0, b]]])
    t = np.array([[[0.0, a], [0.0, 0.0]]])
    p0 = 1.0 / (1.0 + math.exp(a / T))
    q0 = 1.0 / (1.0 + math.exp(b / T))
    assert abs(oracle.acceptance_rate(d, t, T)[0, 0] - (1.0 - abs(p0 - q0))) < 1e-14


@pytest.mark.parametrize("seed,T", [(2, 1.0), (3, 0.7), (4, 1.6)])
def test_acceptance_is_one_minus_total_variation(seed, T):
    rng = np.random.default_rng(seed)
    d = rng.normal(0, 2.0, (4, 3, 2000))
    t = np.concatenate([d + rng.normal(0, 1.0, (4, 3, 2000)), rng.normal(0, 2.0, (4, 1, 2000))], axis=1)
    d[0, 0, :100] = -np.inf  # masked tokens count with probability 0
    a = oracle.acceptance_rate(d, t, T)
    for b in range(4):
        for i in range(3):
            tv = 0.5 * np.abs(_probs(t[b, i], T) - _probs(d[b, i], T)).sum()
            assert abs(a[b, i] - (1.0 - tv)) < 1e-12, (b, i)
    assert np.all((a > 0.0) & (a < 1.0))


@pytest.mark.parametrize("seed,T", [(5, 1.0), (6, 0.7)])
def test_acceptance_equals_enumerated_accept_probability(seed, T):
    rng = np.random.default_rng(seed)
    gamma = 2
    draft = rng.normal(0, 1.5, (gamma, 8))
    target = np.concatenate([draft + rng.normal(0, 0.8, (gamma, 8)), rng.normal(0, 1.5, (1, 8))])
    law, _, _ = _enumerate(draft, target, T)
    a = oracle.acceptance_rate(draft[None], target[None], T)[0]
    p1 = sum(w for (n, _), w in law.items() if n >= 1)
    p2 = sum(w for (n, _), w in law.items() if n >= 2)
    assert abs(p1 - a[0]) < 1e-12
    assert abs(p2 - a[0] * a[1]) < 1e-12


def _definition_draw(logits, T, seed, offset, b, slot):
    w0 = _numpy_block((offset, b, slot, 2), (seed, 0))[0]
    u = (w0 >> 11) / 2.0 ** 53
    q = _probs(logits, T)
    c = np.cumsum(q)
    return int(np.searchsorted(c, u * c[-1], side="right"))


@pytest.mark.parametrize("first_slot", [0, 3])
def test_draws_follow_the_definition_on_stream_2(first_slot):
    rng = np.random.default_rng(8)
    B, R, V, T, seed, offset = 5, 4, 300, 0.9, 11, 6
    logits = rng.normal(0, 2.0, (B, R, V))
    logits[1, 2, 100:] = -np.inf
    x, margin = oracle.draw_tokens(logits, T, seed, offset, first_slot=first_slot)
    assert x.dtype == np.int32 and margin.shape == (B, R)
    for b in range(B):
        for r in range(R):
            assert x[b, r] == _definition_draw(logits[b, r], T, seed, offset, b, first_slot + r), (b, r)
            assert np.isfinite(logits[b, r, x[b, r]])
    assert np.array_equal(oracle.draw_draft_tokens(logits, T, seed, offset),
                          oracle.draw_tokens(logits, T, seed, offset)[0])


def test_one_position_at_a_time_equals_all_at_once():
    rng = np.random.default_rng(9)
    logits = rng.normal(0, 2.0, (3, 5, 200))
    x_all, m_all = oracle.draw_tokens(logits, 1.0, 4, 2)
    for r in range(5):
        x_r, m_r = oracle.draw_tokens(logits[:, r:r + 1], 1.0, 4, 2, first_slot=r)
        assert np.array_equal(x_r[:, 0], x_all[:, r]) and np.array_equal(m_r[:, 0], m_all[:, r])

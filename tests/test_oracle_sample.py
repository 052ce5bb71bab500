"""Pins of the oracle's speculative sampler against the theorem it implements.

The speculative-sampling rule (the two titles the S3R page-3 reference list
cites) makes every emitted token follow the target law: at the first position
P(out_0 = t) = p_0(t); given positions < j accepted, out_j ~ p_j; and
P(n >= k) = prod_{i<k} alpha_i with alpha_i = sum_x min(p_i(x), q_i(x)).

* exact enumeration at vocab 8: every uniform is replaced by the midpoint of
  each interval on which the sampler's behaviour is constant, weighted by the
  interval's length, so the emitted law is computed without Monte Carlo;
* chi-square Monte Carlo at vocab 1024 with the real Philox streams;
* q = p accepts every draft and the bonus follows p_gamma;
* the accepted-length law.
"""
import itertools

import numpy as np
import pytest
from scipy import stats

import oracle


def _softmax(x):
    e = np.exp(x - x.max())
    return e / e.sum()


def _enumerate(draft, target, T=1.0):
    """Exact law of (n, out) by branching over every uniform's constant intervals."""
    gamma, V = draft.shape
    p = [_softmax(target[i] / T) for i in range(gamma + 1)]
    q = [_softmax(draft[i] / T) for i in range(gamma)]
    law = {}

    def intervals_icdf(w):
        c = np.concatenate([[0.0], np.cumsum(w) / w.sum()])
        return [((c[t] + c[t + 1]) / 2, c[t + 1] - c[t]) for t in range(len(w)) if w[t] > 0]

    for xs in itertools.product(range(V), repeat=gamma):
        wx = np.prod([q[i][xs[i]] for i in range(gamma)])
        if wx == 0:
            continue
        # paths: list of (script {(slot, stream): u}, weight)
        paths = [({}, wx)]
        done = []
        for i in range(gamma):
            nxt = []
            r = min(1.0, p[i][xs[i]] / q[i][xs[i]])
            for script, w in paths:
                if r > 0.0:  # p(x) = 0 leaves no accept branch
                    a = dict(script)
                    a[(i, 0)] = r / 2
                    nxt.append((a, w * r))
                if r < 1.0:
                    res = np.maximum(0.0, p[i] - q[i])
                    for u, wu in intervals_icdf(res):
                        s2 = dict(script)
                        s2[(i, 0)] = (r + 1) / 2
                        s2[(i, 1)] = u
                        done.append((s2, w * (1 - r) * wu))
            paths = nxt
        for script, w in paths:
            for u, wu in intervals_icdf(p[gamma]):
                s2 = dict(script)
                s2[(gamma, 1)] = u
                done.append((s2, w * wu))
        for script, w in done:
            out, n, _ = oracle.spec_sample(draft[None], target[None], np.array([xs]), T, 0, 0,
                                           uniform_fn=lambda b, slot, st, s=script: s[(slot, st)])
            key = (int(n[0]), tuple(int(t) for t in out[0] if t >= 0))
            law[key] = law.get(key, 0.0) + w
    return law, p, q


@pytest.mark.parametrize("seed,gamma,T", [(0, 2, 1.0), (1, 3, 1.0), (2, 2, 0.7)])
def test_exact_enumeration_vocab8(seed, gamma, T):
    rng = np.random.default_rng(seed)
    draft = rng.normal(0, 1.5, (gamma, 8))
    target = np.concatenate([draft + rng.normal(0, 0.8, (gamma, 8)), rng.normal(0, 1.5, (1, 8))])
    _check_law(draft, target, T)


def test_exact_enumeration_with_masked_tokens():
    # -inf logits: tokens the drafter never proposes, tokens only the target
    # rules out (their drafts are always rejected) and tokens masked in both.
    rng = np.random.default_rng(7)
    gamma = 2
    draft = rng.normal(0, 1.5, (gamma, 8))
    target = np.concatenate([draft + rng.normal(0, 0.8, (gamma, 8)), rng.normal(0, 1.5, (1, 8))])
    draft[0, [1, 5]] = -np.inf
    draft[1, [0, 7]] = -np.inf
    target[0, [2, 5]] = -np.inf
    target[1, [3]] = -np.inf
    target[2, [6, 7]] = -np.inf
    law = _check_law(draft, target, 1.0)
    for (n, toks), w in law.items():  # no emitted token is impossible under its target
        assert all(np.isfinite(target[j, t]) for j, t in enumerate(toks)) or w == 0.0


def _check_law(draft, target, T):
    gamma = draft.shape[0]
    law, p, q = _enumerate(draft, target, T)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    alpha = [np.minimum(p[i], q[i]).sum() for i in range(gamma)]
    for j in range(gamma + 1):
        # P(out_j = t and positions < j accepted) = prod_{i<j} alpha_i * p_j(t)
        marg = np.zeros(8)
        for (n, toks), w in law.items():
            if n >= j:
                marg[toks[j]] += w
        np.testing.assert_allclose(marg, np.prod(alpha[:j]) * p[j], rtol=1e-10, atol=1e-14)
    for k in range(gamma + 1):
        pk = sum(w for (n, _), w in law.items() if n >= k)
        assert abs(pk - np.prod(alpha[:k])) < 1e-12
    # joint law of the emitted prefix given acceptance of earlier positions
    for (n, toks), w in law.items():
        assert len(toks) == n + 1
    return law


def _mc_batch(V, gamma, B, noise, seed, q_equals_p=False):
    rng = np.random.default_rng(seed)
    d = rng.normal(0, 1.0, (gamma, V))
    t = np.concatenate([d + (0 if q_equals_p else rng.normal(0, noise, (gamma, V))),
                        rng.normal(0, 1.0, (1, V))])
    draft = np.broadcast_to(d, (B, gamma, V))
    target = np.broadcast_to(t, (B, gamma + 1, V))
    return draft, target


def _chi2_pvalue(samples, p, min_expected=5.0):
    n = len(samples)
    counts = np.bincount(samples, minlength=len(p)).astype(float)
    exp = p * n
    order = np.argsort(exp)
    # pool the rarest bins until each pooled bin expects >= min_expected
    obs_b, exp_b, acc_o, acc_e = [], [], 0.0, 0.0
    for i in order:
        acc_o += counts[i]
        acc_e += exp[i]
        if acc_e >= min_expected:
            obs_b.append(acc_o)
            exp_b.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0:
        obs_b[-1] += acc_o
        exp_b[-1] += acc_e
    return stats.chisquare(obs_b, exp_b).pvalue


def test_monte_carlo_chi_square_vocab1024():
    V, gamma, B = 1024, 2, 6000
    draft, target = _mc_batch(V, gamma, B, 0.6, seed=11)
    x = oracle.draw_draft_tokens(draft, 1.0, seed=3, offset=0)
    out, n, _ = oracle.spec_sample(draft, target, x, 1.0, seed=3, offset=0)
    p0 = _softmax(target[0, 0])
    assert _chi2_pvalue(out[:, 0], p0) > 1e-3
    p1 = _softmax(target[0, 1])
    assert _chi2_pvalue(out[n >= 1, 1], p1) > 1e-3
    # the draft tokens themselves follow q (pins the stream-2 drafter draws)
    assert _chi2_pvalue(x[:, 0], _softmax(draft[0, 0])) > 1e-3


def test_q_equals_p_accepts_everything():
    V, gamma, B = 512, 3, 3000
    draft, target = _mc_batch(V, gamma, B, 0.0, seed=12, q_equals_p=True)
    x = oracle.draw_draft_tokens(draft, 1.0, seed=5, offset=2)
    out, n, dec = oracle.spec_sample(draft, target, x, 1.0, seed=5, offset=2)
    assert np.all(n == gamma)
    assert np.array_equal(out[:, :gamma], x)
    assert _chi2_pvalue(out[:, gamma], _softmax(target[0, gamma])) > 1e-3


def test_accepted_length_law():
    V, gamma, B = 256, 4, 8000
    draft, target = _mc_batch(V, gamma, B, 1.2, seed=13)
    x = oracle.draw_draft_tokens(draft, 1.0, seed=9, offset=1)
    _, n, _ = oracle.spec_sample(draft, target, x, 1.0, seed=9, offset=1)
    alpha = [np.minimum(_softmax(target[0, i]), _softmax(draft[0, i])).sum() for i in range(gamma)]
    # the oracle's acceptance rate is the same law's per-position factor
    np.testing.assert_allclose(oracle.acceptance_rate(draft[:1], target[:1], 1.0)[0], alpha, rtol=0, atol=1e-12)
    for k in range(1, gamma + 1):
        expect = np.prod(alpha[:k])
        got = np.mean(n >= k)
        sd = np.sqrt(expect * (1 - expect) / B)
        assert abs(got - expect) < 5 * sd + 1e-9, (k, got, expect)


def test_icdf_edges():
    assert oracle.icdf([0.0, 1.0, 0.0], 0.0)[0] == 1
    assert oracle.icdf([0.5, 0.5], 0.5)[0] == 1      # strict '>' at the boundary
    assert oracle.icdf([0.5, 0.5], 0.4999)[0] == 0
    assert oracle.icdf([1.0, 0.0, 2.0, 0.0], 0.999999)[0] == 2
    t, m = oracle.icdf([0.25, 0.25, 0.5], 0.5)
    assert t == 2 and m == 0.0


def test_output_format():
    rng = np.random.default_rng(3)
    d = rng.normal(0, 2, (5, 4, 64))
    t = np.concatenate([d + rng.normal(0, 2, (5, 4, 64)), rng.normal(0, 2, (5, 1, 64))], axis=1)
    x = oracle.draw_draft_tokens(d, 1.0, 0, 0)
    out, n, dec = oracle.spec_sample(d, t, x, 1.0, 0, 0)
    for b in range(5):
        assert np.all(out[b, :n[b]] == x[b, :n[b]])
        assert 0 <= out[b, n[b]] < 64
        assert np.all(out[b, n[b] + 1:] == -1)
        assert dec[b][-1][0] == n[b] and dec[b][-1][1] == "draw"

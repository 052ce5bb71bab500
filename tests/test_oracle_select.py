"""Pins of the oracle's page bounds and page selection.

* bounds: the score of a page bounds scale*q.k_t of every token in it (brute
  force over all tokens), and is exact for a one-token page;
* ranking: equals an independent numpy.lexsort ranking of the same scores;
* ties (q = 0, all scores equal) keep the lowest page indices;
* a budget covering every page returns 0..n-1;
* planted high-norm pages are always selected;
* permuting the physical pool does not change the logical selection.
"""
import numpy as np
import pytest
import torch

import oracle
from s3r_inputs import make_workload
from tests.oracle_io import f64, i32


def _wl(seed=0, ctx=(200, 75, 16), kv="bf16", D=64, heavy=0, G=2):
    return make_workload(dict(B=len(ctx), Hq=2 * G, Hkv=2, D=D, L=None, P=16, budget=64,
                              gamma=2, V=16, kv_dtype=kv, draft_sd=1.0, noise_sd=0.5,
                              temperature=1.0, heavy_pages=heavy), seed=seed, ctx=list(ctx),
                         with_logits=False)


def test_bounds_are_min_max_and_bound_every_logit():
    wl = _wl(seed=1)
    K, pt, L = f64(wl.k_pool), i32(wl.page_table), i32(wl.seq_lens[1])
    bounds = oracle.page_bounds(K, pt, L)
    q = f64(wl.draft_q(1))
    scale = 1 / 8
    G = 2
    for b in range(len(L)):
        for h in range(2):
            sc = oracle.page_scores(bounds, q, pt, L, scale, b, h)
            for t in range(L[b]):
                kt = oracle.key_row(K, pt, b, h, t)
                best = max(scale * float(q[b, g] @ kt) for g in range(h * G, h * G + G))
                assert sc[t // 16] >= best - 1e-12
            # every stored bound is attained by some token of the page
            for j in range(oracle.n_pages(L[b], 16)):
                toks = np.stack([oracle.key_row(K, pt, b, h, t)
                                 for t in range(16 * j, min(16 * j + 16, L[b]))])
                assert np.all(np.any(toks == bounds[pt[b, j], h, 0], axis=0))
                assert np.all(np.any(toks == bounds[pt[b, j], h, 1], axis=0))
                assert np.all(bounds[pt[b, j], h, 0] <= bounds[pt[b, j], h, 1])


def test_one_token_page_score_is_the_exact_logit():
    wl = _wl(seed=2, ctx=(33,))  # tail page holds exactly one token
    K, pt, L = f64(wl.k_pool), i32(wl.page_table), i32(wl.seq_lens[0])
    bounds = oracle.page_bounds(K, pt, L)
    q = f64(wl.draft_q(0))
    sc = oracle.page_scores(bounds, q, pt, L, 0.5, 0, 1)
    kt = oracle.key_row(K, pt, 0, 1, 32)
    exact = max(0.5 * float(q[0, g] @ kt) for g in (2, 3))
    assert abs(sc[2] - exact) <= 1e-12 * max(1.0, abs(exact))


@pytest.mark.parametrize("budget", [16, 48, 80, 160])
def test_selection_equals_lexsort_ranking(budget):
    wl = _wl(seed=3, ctx=(300, 130, 40))
    K, pt, L = f64(wl.k_pool), i32(wl.page_table), i32(wl.seq_lens[2])
    bounds = oracle.page_bounds(K, pt, L)
    q = f64(wl.draft_q(2))
    sel, nsel, scores = oracle.page_select(bounds, q, pt, L, budget, 0.125)
    k = budget // 16
    for b in range(len(L)):
        n = oracle.n_pages(L[b], 16)
        assert nsel[b] == min(k, n)
        for h in range(2):
            if k >= n:
                assert list(sel[b, h, :n]) == list(range(n))
                assert np.all(sel[b, h, n:] == -1)
                continue
            sc = scores[(b, h)]
            order = np.lexsort((np.arange(n), -sc))  # score desc, then index asc
            assert list(sel[b, h]) == sorted(order[:k].tolist())


def test_ties_keep_lowest_indices():
    wl = _wl(seed=4, ctx=(160,))
    K, pt, L = f64(wl.k_pool), i32(wl.page_table), i32(wl.seq_lens[0])
    bounds = oracle.page_bounds(K, pt, L)
    q = np.zeros_like(f64(wl.draft_q(0)))
    sel, _, _ = oracle.page_select(bounds, q, pt, L, 64, 0.125)
    assert np.all(sel == np.array([0, 1, 2, 3]))


def test_heavy_pages_always_selected():
    wl = _wl(seed=5, ctx=(1000, 777), D=64, heavy=4)
    K, pt, L = f64(wl.k_pool), i32(wl.page_table), i32(wl.seq_lens[0])
    bounds = oracle.page_bounds(K, pt, L)
    q = f64(wl.draft_q(0))
    sel, _, _ = oracle.page_select(bounds, q, pt, L, 128, 0.125)
    for b in range(2):
        for h in range(2):
            assert set(wl.heavy[b].tolist()) <= set(sel[b, h].tolist())


def test_selection_is_invariant_to_pool_permutation():
    wl = _wl(seed=6, ctx=(120, 90))
    K, pt, L = f64(wl.k_pool), i32(wl.page_table), i32(wl.seq_lens[0])
    q = f64(wl.draft_q(0))
    sel1, _, _ = oracle.page_select(oracle.page_bounds(K, pt, L), q, pt, L, 48, 0.1)
    perm = np.random.default_rng(0).permutation(K.shape[0])
    inv = np.argsort(perm)
    K2 = K[perm]
    pt2 = inv[pt]
    sel2, _, _ = oracle.page_select(oracle.page_bounds(K2, pt2, L), q, pt2, L, 48, 0.1)
    assert np.array_equal(sel1, sel2)

"""Pins of the oracle's once-per-round page selection (forced tail pages).

* forced pages: hand-worked cases of "the pages holding positions
  seq_len - 1 .. seq_len + gamma - 2", including empty, page-crossing and
  table-width-clipped rounds;
* the kept set: every forced page, ascending, -1 padded, counted;
* the scored part: equals an independent numpy.lexsort ranking of the
  candidate pages, and no dropped candidate outranks a kept one;
* gamma = 1 with the tail page already a top page reduces to page_select;
* a budget covering every page keeps them all plus the round's future page;
* a budget below the forced pages is refused.
"""
import numpy as np
import pytest

import oracle
from s3r_inputs import make_workload
from tests.oracle_io import f64, i32


@pytest.mark.parametrize("L,gamma,maxp,expect", [
    (33, 1, 8, [2]),        # one query at position 32: page 2
    (33, 6, 8, [2]),        # positions 32..37 stay in page 2
    (32, 2, 8, [1, 2]),     # positions 31, 32 cross into page 2
    (16, 16, 8, [0, 1]),    # positions 15..30
    (48, 16, 8, [2, 3]),    # positions 47..62
    (1, 4, 8, [0]),         # positions 0..3
    (0, 3, 8, [0]),         # no context yet: positions 0..1
    (0, 1, 8, []),          # the only query sits at position -1
    (32, 2, 2, [1]),        # page 2 lies past the table width
])
def test_forced_pages_hand_worked(L, gamma, maxp, expect):
    assert oracle.round_forced_pages(L, gamma, 16, maxp) == expect


def _wl(seed, ctx, D=64, G=2, heavy=0):
    return make_workload(dict(B=len(ctx), Hq=2 * G, Hkv=2, D=D, L=None, P=16, budget=64,
                              gamma=2, V=16, kv_dtype="bf16", draft_sd=1.0, noise_sd=0.5,
                              temperature=1.0, heavy_pages=heavy), seed=seed, ctx=list(ctx),
                         with_logits=False)


def _inputs(wl, step=0):
    K, pt, L = f64(wl.k_pool), i32(wl.page_table), i32(wl.seq_lens[step])
    return oracle.page_bounds(K, pt, L), f64(wl.draft_q(step)), pt, L


@pytest.mark.parametrize("seed,ctx,budget,gamma", [
    (0, (200, 75, 16), 64, 2),
    (1, (511, 129, 300), 96, 6),
    (2, (1000, 47), 128, 16),
    (3, (257, 64, 33), 32, 3),
])
def test_kept_set_is_forced_plus_best_candidates(seed, ctx, budget, gamma):
    wl = _wl(seed, ctx, heavy=2)
    bounds, q, pt, L = _inputs(wl)
    scale = 0.125
    sel, nsel, scores = oracle.page_select_round(bounds, q, pt, L, budget, gamma, scale)
    k = budget // 16
    for b in range(len(ctx)):
        n = oracle.n_pages(int(L[b]), 16)
        forced = oracle.round_forced_pages(int(L[b]), gamma, 16, pt.shape[1])
        cands = np.array([j for j in range(n) if j not in forced], dtype=np.int64)
        rest = k - len(forced)
        for h in range(2):
            row = sel[b, h]
            kept = row[row >= 0]
            assert np.all(row[len(kept):] == -1) and np.all(np.diff(kept) > 0)
            assert len(kept) == nsel[b] == len(forced) + min(rest, len(cands))
            assert set(forced) <= set(kept.tolist())
            chosen = sorted(set(kept.tolist()) - set(forced))
            if rest >= len(cands):
                assert chosen == cands.tolist()
                continue
            sc = oracle.page_scores(bounds, q, pt, L, scale, b, h)[cands]
            ranked = cands[np.lexsort((cands, -sc))][:rest]
            assert chosen == sorted(ranked.tolist())
            # no dropped candidate outranks a kept one
            kept_sc = {j: s for j, s in zip(cands, sc)}
            if chosen:
                worst = min((kept_sc[j], -j) for j in chosen)
                assert all((kept_sc[j], -j) < worst for j in cands if j not in chosen)


def test_gamma_one_with_a_top_tail_page_equals_page_select():
    wl = _wl(4, (300, 190, 77))
    # make every sequence's tail page the highest-scoring page
    for b, L in enumerate(wl.ctx):
        phys = int(wl.page_table[b, (int(L) - 1) // 16])
        wl.k_pool[phys] = wl.k_pool[phys] * 64
    bounds, q, pt, L = _inputs(wl)
    for budget in (32, 64, 160):
        a = oracle.page_select_round(bounds, q, pt, L, budget, 1, 0.125)
        p = oracle.page_select(bounds, q, pt, L, budget, 0.125)
        assert np.array_equal(a[0], p[0]) and np.array_equal(a[1], p[1])


def test_full_budget_keeps_every_page_and_the_future_tail():
    wl = _wl(5, (64, 40))  # 64 tokens: the round's second query opens page 4
    bounds, q, pt, L = _inputs(wl)
    sel, nsel, _ = oracle.page_select_round(bounds, q, pt, L, 16 * 16, 3, 0.125)
    assert sel[0, 0, :6].tolist() == [0, 1, 2, 3, 4, -1] and nsel[0] == 5
    assert sel[1, 1, :4].tolist() == [0, 1, 2, -1] and nsel[1] == 3


def test_budget_below_the_forced_pages_is_refused():
    wl = _wl(6, (32,))
    bounds, q, pt, L = _inputs(wl)
    with pytest.raises(ValueError):
        oracle.page_select_round(bounds, q, pt, L, 16, 2, 0.125)  # k = 1, pages 1 and 2 forced

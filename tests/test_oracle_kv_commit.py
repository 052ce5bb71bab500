"""Pins of the oracle's KV commit (append + bounds maintenance + rollback).

* written rows read back at their positions through the pool layout
  accessors, and nothing else in either pool changes;
* every refreshed bound is attained by a valid token of its page and bounds
  all of them (the page_bounds invariant), so rows past the committed length
  (a rollback) cannot move any bound: planting huge values there changes
  nothing;
* pages outside the touched range keep their bounds;
* appending rows one at a time equals appending them at once;
* rows past the page table, or in a page whose table entry is negative
  (unallocated), are dropped;
* a pure rollback (no rows) shrinks the tail page's bounds to its remaining
  tokens, and a rollback below the page the rows went to re-bounds the new
  tail page.
"""
import numpy as np
import pytest

import oracle
from s3r_inputs import make_workload
from tests.oracle_io import f64, i32


def _setup(seed, ctx, gamma=5, D=64, Hkv=2):
    wl = make_workload(dict(B=len(ctx), Hq=2 * Hkv, Hkv=Hkv, D=D, L=None, P=16, budget=64,
                            gamma=gamma, V=16, kv_dtype="f32", draft_sd=1.0, noise_sd=0.5,
                            temperature=1.0, heavy_pages=0), seed=seed, ctx=list(ctx),
                       with_logits=False)
    K, V, pt = f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table)
    L0 = i32(wl.seq_lens[0])
    bounds = oracle.page_bounds(K, pt, L0)
    return wl, K, V, pt, L0, bounds


def _new_rows(seed, B, count, Hkv, D):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, count, Hkv, D)), rng.standard_normal((B, count, Hkv, D))


@pytest.mark.parametrize("ctx,count,accepted", [
    ((40, 17, 64), 6, (5, 0, 2)),     # verify-sized writes, partial accepts
    ((15, 16, 200), 3, (2, 2, 2)),    # writes that open a page
    ((33, 1, 90), 1, (0, 0, 0)),      # one row, nothing kept beyond it
])
def test_rows_land_and_bounds_follow(ctx, count, accepted):
    wl, K, V, pt, L0, bounds = _setup(1, ctx)
    B, Hkv, D = len(ctx), 2, 64
    kn, vn = _new_rows(2, B, count, Hkv, D)
    first = L0 - 1
    Lc = first + 1 + np.array(accepted)          # committed: the first row plus the accepts
    K2, V2, B2 = oracle.kv_commit(K, V, pt, kn, vn, first, Lc, bounds)
    touched = np.zeros(K.shape[:1] + K.shape[2:3], dtype=bool)  # [phys][slot]
    for b in range(B):
        for i in range(count):
            t = int(first[b]) + i
            for h in range(Hkv):
                assert np.array_equal(oracle.key_row(K2, pt, b, h, t), kn[b, i, h])
                assert np.array_equal(oracle.value_row(V2, pt, b, h, t), vn[b, i, h])
            touched[pt[b, t // 16], t % 16] = True
    keep = ~touched
    assert np.array_equal(K2.transpose(0, 2, 1, 3)[keep], K.transpose(0, 2, 1, 3)[keep])
    assert np.array_equal(V2.transpose(0, 3, 1, 2)[keep], V.transpose(0, 3, 1, 2)[keep])
    for b in range(B):
        L = int(Lc[b])
        lo = min(int(first[b]), L - 1) // 16
        for j in range(oracle.n_pages(L, 16)):
            phys = pt[b, j]
            if j < lo:
                assert np.array_equal(B2[phys], bounds[phys], equal_nan=True)
                continue
            for h in range(Hkv):
                rows = np.stack([oracle.key_row(K2, pt, b, h, t)
                                 for t in range(16 * j, min(16 * j + 16, L))])
                assert np.all(rows >= B2[phys, h, 0]) and np.all(rows <= B2[phys, h, 1])
                assert np.all(np.any(rows == B2[phys, h, 0], axis=0))
                assert np.all(np.any(rows == B2[phys, h, 1], axis=0))


def test_rolled_back_rows_do_not_move_bounds():
    wl, K, V, pt, L0, bounds = _setup(3, (50, 31))
    kn, vn = _new_rows(4, 2, 5, 2, 64)
    first = L0 - 1
    Lc = first + 2                                   # keep two of the five rows
    _, _, a = oracle.kv_commit(K, V, pt, kn, vn, first, Lc, bounds)
    kn2 = kn.copy()
    kn2[:, 2:] = 1e6 * np.sign(kn2[:, 2:])           # the rejected rows
    _, _, c = oracle.kv_commit(K, V, pt, kn2, vn, first, Lc, bounds)
    assert np.array_equal(a, c, equal_nan=True)


def test_one_row_at_a_time_equals_all_at_once():
    wl, K, V, pt, L0, bounds = _setup(5, (47, 16, 100))
    kn, vn = _new_rows(6, 3, 4, 2, 64)
    first = L0 - 1
    all_at_once = oracle.kv_commit(K, V, pt, kn, vn, first, first + 4, bounds)
    K1, V1, B1 = K, V, bounds
    for i in range(4):
        K1, V1, B1 = oracle.kv_commit(K1, V1, pt, kn[:, i:i + 1], vn[:, i:i + 1], first + i,
                                      first + i + 1, B1)
    for x, y in zip(all_at_once, (K1, V1, B1)):
        assert np.array_equal(x, y, equal_nan=True)


def test_rows_past_the_table_are_dropped():
    wl, K, V, pt, L0, bounds = _setup(7, (60,), gamma=2)   # table: ceil(62 / 16) = 4 pages
    kn, vn = _new_rows(8, 1, 8, 2, 64)
    first = np.array([60])
    K2, V2, _ = oracle.kv_commit(K, V, pt, kn, vn, first, np.array([64]), bounds)
    for i in range(4):
        assert np.array_equal(oracle.key_row(K2, pt, 0, 1, 60 + i), kn[0, i, 1])
    assert np.array_equal(K2[pt[0, 0]], K[pt[0, 0]])


def test_pure_rollback_shrinks_the_tail_page():
    wl, K, V, pt, L0, bounds = _setup(9, (45,))
    kn, vn = np.zeros((1, 0, 2, 64)), np.zeros((1, 0, 2, 64))
    _, _, b2 = oracle.kv_commit(K, V, pt, kn, vn, np.array([44]), np.array([35]), bounds)
    rows = np.stack([oracle.key_row(K, pt, 0, 0, t) for t in range(32, 35)])
    assert np.array_equal(b2[pt[0, 2], 0, 0], rows.min(axis=0))
    assert np.array_equal(b2[pt[0, 2], 0, 1], rows.max(axis=0))
    assert np.array_equal(b2[pt[0, 0]], bounds[pt[0, 0]])


def test_rows_in_an_unallocated_page_are_dropped():
    wl, K, V, pt, L0, bounds = _setup(11, (30,), gamma=6)   # pages 0, 1 and 2 (positions < 36)
    pt = pt.copy()
    pt[0, 2] = -1                                            # page 2 not allocated
    kn, vn = _new_rows(12, 1, 5, 2, 64)
    K2, V2, B2 = oracle.kv_commit(K, V, pt, kn, vn, np.array([29]), np.array([33]), bounds)
    # Positions 29..31 land in page 1; nothing else anywhere in either pool changes.
    Ke, Ve = K.copy(), V.copy()
    for i in range(3):
        Ke[pt[0, 1], :, 13 + i, :] = kn[0, i]
        Ve[pt[0, 1], :, :, 13 + i] = vn[0, i]
    assert np.array_equal(K2, Ke) and np.array_equal(V2, Ve)


def test_rollback_across_a_page_boundary_rebounds_the_new_tail_page():
    # 45 tokens, three rows written at 44..46, then only 30 kept: the new tail
    # is page 1 (tokens 16..29), below the page the rows went to.
    wl, K, V, pt, L0, bounds = _setup(13, (45,))
    kn, vn = _new_rows(14, 1, 3, 2, 64)
    K2, _, b2 = oracle.kv_commit(K, V, pt, kn, vn, np.array([44]), np.array([30]), bounds)
    for h in range(2):
        rows = np.stack([oracle.key_row(K2, pt, 0, h, t) for t in range(16, 30)])
        assert np.array_equal(b2[pt[0, 1], h, 0], rows.min(axis=0))
        assert np.array_equal(b2[pt[0, 1], h, 1], rows.max(axis=0))
    assert np.array_equal(b2[pt[0, 2]], bounds[pt[0, 2]])   # no valid token left: kept
    assert np.array_equal(b2[pt[0, 0]], bounds[pt[0, 0]])

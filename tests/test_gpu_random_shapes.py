"""GPU parity over seeded random shapes inside the supported range.

Each case draws the shape from a fixed seed:
- G in 1..8 and Hkv in {1, 2, 3, 4, 8}, D in {64, 128}, bf16 or fp32 KV;
- 1..6 sequences of 1..3000 tokens, a budget of 2..48 pages, gamma with G * (gamma + 1) <= 64.

Each case runs every attention-side entry point and compares it with the oracle:
- page bounds, page selection and the sparse draft over that selection;
- the one-call draft step (whichever of its paths the shape takes);
- the once-per-round selection and the dense verify.

The split sizes, wave counts and combine paths these shapes select are the ones the
fixed cases do not enumerate. Random KV commits (rollbacks, unallocated pages) and
random sampling rounds (vocabularies of 1..20000, gamma up to 16, several
temperatures) follow. Tolerances are those of test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
import self_sparse_speculative_paged_amd as s3r
from s3r_inputs import make_workload
from tests.oracle_io import f64, i32
from tests.parity import check_pages

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _shape(seed):
    rng = np.random.default_rng(1000 + seed)
    G = int(rng.integers(1, 9))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    D = int(rng.choice([64, 128]))
    kv = "f32" if rng.random() < 0.25 else "bf16"
    B = int(rng.integers(1, 7))
    ctx = [int(x) for x in rng.integers(1, 3001, size=B)]
    gamma = int(rng.integers(1, min(16, 64 // G - 1) + 1))
    budget = 16 * int(rng.integers(2, 49))  # the round needs at least two pages
    return G, Hkv, D, kv, ctx, gamma, budget


def _attn_ok(got, ref, kv):
    got = got.float().cpu().numpy().astype(np.float64)
    ok = ~np.isnan(ref)
    if kv == "f32":
        scale = max(np.max(np.abs(ref[ok])), 1e-30)
        assert np.max(np.abs(got[ok] - ref[ok])) / scale <= 1e-5
    else:
        assert np.max(np.abs(got[ok] - ref[ok])) <= 1e-2


@pytest.mark.parametrize("seed", range(48))
def test_random_shape_matches_oracle(seed):
    G, Hkv, D, kv, ctx, gamma, budget = _shape(seed)
    print(f"random shape {seed}: G={G} Hkv={Hkv} D={D} kv={kv} ctx={ctx} gamma={gamma} budget={budget}",
          flush=True)
    cfg = dict(B=len(ctx), Hq=G * Hkv, Hkv=Hkv, D=D, L=None, P=16, budget=budget, gamma=gamma, V=64,
               kv_dtype=kv, draft_sd=2.0, noise_sd=0.7, temperature=1.0, heavy_pages=0)
    wl = make_workload(cfg, device="cpu", seed=seed, ctx=ctx, with_logits=False)
    k_pool, v_pool, pt = wl.k_pool.to(DEV), wl.v_pool.to(DEV), wl.page_table.to(DEV)
    seq = [s.to(DEV) for s in wl.seq_lens]
    K, V, P = f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table)
    scale = 1.0 / np.sqrt(D)
    k = budget // 16
    hint = sum(-(-(L + gamma) // 16) for L in ctx) if seed % 2 else 0
    kvc = lambda j: s3r.PagedKVCache(k_pool, v_pool, pt, seq[j], G * Hkv, total_pages_hint=hint)

    # bounds, select and draft at step 0
    L0 = i32(wl.seq_lens[0])
    bounds = torch.zeros((k_pool.shape[0], Hkv, 2, D), dtype=k_pool.dtype, device=DEV)
    s3r.page_bounds_update(kvc(0), bounds)
    q0 = wl.draft_q(0).to(DEV)
    sel, nsel = s3r.page_select(kvc(0), bounds, q0, budget, scale)
    d_out = s3r.sparse_draft_attn(kvc(0), q0, sel, scale)
    torch.cuda.synchronize()
    rb = oracle.page_bounds(K, P, L0)
    used = ~np.isnan(rb[:, 0, 0, 0])
    assert np.array_equal(f64(bounds)[used], rb[used])
    rsel, rn, rsc = oracle.page_select(rb, f64(wl.draft_q(0)), P, L0, budget, scale)
    check_pages(i32(sel), i32(nsel), rsel, rn, rsc, k)
    _attn_ok(d_out, oracle.sparse_draft_attn(f64(wl.draft_q(0)), K, V, P, L0, i32(sel), scale), kv)

    # the one-call draft step at step 1 (bounds refreshed from its first position)
    L1 = i32(wl.seq_lens[1])
    q1 = wl.draft_q(1).to(DEV)
    out1, sel1, nsel1 = s3r.sparse_draft_step(kvc(1), bounds, q1, budget, scale,
                                              refresh_from=(seq[1] - 1).contiguous())
    torch.cuda.synchronize()
    rb1 = oracle.page_bounds(K, P, L1)
    rsel1, rn1, rsc1 = oracle.page_select(rb1, f64(wl.draft_q(1)), P, L1, budget, scale)
    check_pages(i32(sel1), i32(nsel1), rsel1, rn1, rsc1, k)
    _attn_ok(out1, oracle.sparse_draft_attn(f64(wl.draft_q(1)), K, V, P, L1, i32(sel1), scale), kv)

    # the once-per-round selection at step 0
    s3r.page_bounds_update(kvc(0), bounds)
    _, selr, nselr = s3r.sparse_draft_round(kvc(0), bounds, q0, budget, gamma, scale,
                                            refresh_from=(seq[0] - 1).contiguous())
    torch.cuda.synchronize()
    rr, rrn, rrsc = oracle.page_select_round(rb, f64(wl.draft_q(0)), P, L0, budget, gamma, scale)
    assert np.array_equal(i32(nselr), rrn)
    for b in range(len(ctx)):
        forced = oracle.round_forced_pages(int(L0[b]), gamma, 16, P.shape[1])
        for h in range(Hkv):
            g = [int(x) for x in i32(selr)[b, h] if x >= 0]
            r = [int(x) for x in rr[b, h] if x >= 0]
            assert set(forced) <= set(g) and len(g) == len(r) and g == sorted(g)
            if g != r:
                sc = rrsc[(b, h)]
                kth = sorted(sc.values(), reverse=True)[k - len(forced) - 1]
                assert all(abs(sc[j] - kth) <= 1e-4 for j in set(g) ^ set(r)), (b, h)

    # dense verify of gamma + 1 queries
    Lv = i32(wl.seq_lens[gamma])
    v_out = s3r.dense_verify_attn(kvc(gamma), wl.q_verify.to(DEV), scale)
    torch.cuda.synchronize()
    _attn_ok(v_out, oracle.dense_verify_attn(f64(wl.q_verify), K, V, P, Lv, scale), kv)


@pytest.mark.parametrize("seed", range(16))
def test_random_kv_commit_matches_oracle(seed):
    """Random commits: rows from a random first position, some past the
    committed length (rolled back), an occasional unallocated page; pools and
    bounds bit-exact against the oracle."""
    rng = np.random.default_rng(2000 + seed)
    Hkv = int(rng.choice([1, 2, 3, 8]))
    D = int(rng.choice([64, 128]))
    kv = "f32" if rng.random() < 0.3 else "bf16"
    B = int(rng.integers(1, 6))
    ctx = [int(x) for x in rng.integers(1, 800, size=B)]
    count = int(rng.integers(0, 18))
    slack = count + 2
    print(f"random commit {seed}: Hkv={Hkv} D={D} kv={kv} ctx={ctx} count={count}", flush=True)
    cfg = dict(B=B, Hq=Hkv, Hkv=Hkv, D=D, L=None, P=16, budget=64, gamma=slack, V=64, kv_dtype=kv,
               draft_sd=2.0, noise_sd=0.7, temperature=1.0, heavy_pages=0)
    wl = make_workload(cfg, device="cpu", seed=seed, ctx=ctx, with_logits=False)
    pt = wl.page_table.clone()
    if rng.random() < 0.5:  # one unallocated page past some sequence's start
        b = int(rng.integers(0, B))
        j = int(rng.integers(0, pt.shape[1]))
        pt[b, j] = -1
    first = np.array([max(0, L - 1 - int(rng.integers(0, 3))) for L in ctx], dtype=np.int32)
    committed = np.array([max(0, int(f) + int(rng.integers(-3, count + 2))) for f in first], dtype=np.int32)
    dt = wl.k_pool.dtype
    g = torch.Generator().manual_seed(seed)
    k_new = torch.randn((B, count, Hkv, D), generator=g).to(dt)
    v_new = torch.randn((B, count, Hkv, D), generator=g).to(dt)
    k_pool, v_pool, ptd = wl.k_pool.to(DEV), wl.v_pool.to(DEV), pt.to(DEV)
    kvc0 = s3r.PagedKVCache(k_pool, v_pool, ptd, torch.from_numpy(np.array(ctx, dtype=np.int32)).to(DEV), Hkv)
    bounds = torch.zeros((k_pool.shape[0], Hkv, 2, D), dtype=dt, device=DEV)
    s3r.page_bounds_update(s3r.PagedKVCache(k_pool, v_pool, wl.page_table.to(DEV), kvc0.seq_lens, Hkv), bounds)
    torch.cuda.synchronize()
    K0, V0, B0 = f64(wl.k_pool), f64(wl.v_pool), f64(bounds)
    rK, rV, rB = oracle.kv_commit(K0, V0, i32(pt), f64(k_new), f64(v_new), first, committed, B0)
    kvc = s3r.PagedKVCache(k_pool, v_pool, ptd, torch.from_numpy(committed).to(DEV), Hkv)
    s3r.kv_commit(kvc, k_new.to(DEV), v_new.to(DEV), torch.from_numpy(first).to(DEV), bounds)
    torch.cuda.synchronize()
    assert np.array_equal(f64(k_pool), rK) and np.array_equal(f64(v_pool), rV)
    assert np.array_equal(f64(bounds), rB, equal_nan=True)


@pytest.mark.parametrize("seed", range(12))
def test_random_spec_sample_matches_oracle(seed):
    rng = np.random.default_rng(3000 + seed)
    B = int(rng.integers(1, 33))
    gamma = int(rng.integers(1, 17))
    V = int(rng.integers(1, 20000))
    T = float(rng.choice([0.5, 0.8, 1.0, 1.3]))
    noise = float(rng.choice([0.0, 0.3, 1.0, 2.5]))
    print(f"random sample {seed}: B={B} gamma={gamma} V={V} T={T} noise={noise}", flush=True)
    g = torch.Generator().manual_seed(seed)
    d = torch.randn((B, gamma, V), generator=g) * 2.0
    t = torch.cat([d + torch.randn((B, gamma, V), generator=g) * noise,
                   torch.randn((B, 1, V), generator=g) * 2.0], dim=1)
    x = oracle.draw_draft_tokens(d.double().numpy(), T, seed=seed, offset=0)
    out, n = s3r.spec_sample(d.to(DEV), t.to(DEV), torch.from_numpy(x).to(DEV).int(), T, seed=seed, offset=5)
    torch.cuda.synchronize()
    ro, rn, dec = oracle.spec_sample(d.double().numpy(), t.double().numpy(), x, T, seed, 5)
    from tests.parity import check_tokens
    full = check_tokens(i32(out), i32(n), ro, rn, dec)
    assert full >= B // 2, (full, B)

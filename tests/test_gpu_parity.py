"""GPU parity: every libs3r entry point against the fp64 CPU oracle on the same
seeded inputs, through the C ABI.

Tolerances: page ids bit-exact outside a 1e-4 score tie window; tokens and
accepted lengths bit-exact outside a 1e-6 decision window; attention max-abs
1e-2 for bf16 KV (fp32 accumulation) and norm-wise relative 1e-5 for fp32 KV.
Sizes span several KV tiles, split-KV partitions and ragged tails.
"""
import numpy as np
import pytest
import torch

import oracle
import self_sparse_speculative_paged_amd as s3r
from s3r_inputs import make_workload
from tests.oracle_io import f64, i32
from tests.parity import check_pages, check_tokens

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cfg(kv="bf16", D=128, G=4, Hkv=2, gamma=4, budget=64, V=512, heavy=0):
    return dict(B=None, Hq=G * Hkv, Hkv=Hkv, D=D, L=None, P=16, budget=budget, gamma=gamma, V=V,
                kv_dtype=kv, draft_sd=2.0, noise_sd=0.7, temperature=1.0, heavy_pages=heavy)


def _make(cfg, ctx, seed=0, with_logits=False):
    cfg = dict(cfg, B=len(ctx))
    wl = make_workload(cfg, device="cpu", seed=seed, ctx=ctx, with_logits=with_logits)
    for name in ("k_pool", "v_pool", "page_table", "q_verify", "draft_logits", "target_logits",
                 "draft_tokens"):
        t = getattr(wl, name)
        if t is not None:
            setattr(wl, name, t.to(DEV))
    wl.seq_lens = [s.to(DEV) for s in wl.seq_lens]
    return wl


def _kv(wl, step, hint=0):
    return s3r.PagedKVCache(wl.k_pool, wl.v_pool, wl.page_table, wl.seq_lens[step],
                            wl.cfg["Hq"], total_pages_hint=hint)


def _check_attn(got, ref, kv):
    got = got.float().cpu().numpy().astype(np.float64)
    if kv == "f32":
        err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
        assert err <= 1e-5, err
    else:
        err = np.max(np.abs(got - ref))
        assert err <= 1e-2, err
    return err


VERIFY_CASES = [
    # kv, D, G, Hkv, gamma, ctx
    ("f32", 64, 2, 2, 4, (512, 300)),            # the tiny fp32 shape, ragged second sequence
    ("f32", 128, 4, 2, 6, (250, 17)),
    ("bf16", 128, 2, 2, 4, (700, 33, 1)),        # 10 rows: one MFMA row block
    ("bf16", 128, 4, 2, 6, (1000, 515, 129)),    # 28 rows: two row blocks (Qwen3-8B heads)
    ("bf16", 128, 4, 2, 8, (777, 64)),           # 36 rows: three row blocks
    ("bf16", 64, 8, 1, 7, (400, 95)),            # 64 rows: four row blocks, D=64
    ("bf16", 128, 8, 1, 7, (300, 77)),           # 64 rows at D=128: K/V staged through LDS
    ("bf16", 64, 2, 3, 3, (48, 2049)),
    # query groups that are not a power of two
    ("bf16", 128, 3, 2, 5, (500, 90)),           # 18 rows: two row blocks
    ("bf16", 64, 5, 2, 2, (300, 33)),            # 15 rows: one row block
    ("bf16", 128, 7, 1, 8, (260, 40)),           # 63 rows: four row blocks
    ("bf16", 128, 4, 2, 8, (200, 9, 31)),         # 36 rows, one split per (sequence, kv head)
    ("bf16", 128, 5, 3, 7, (3000, 1500, 17, 260)),  # 40 rows, many splits, odd page counts
    # four row blocks at D=128: K/V staged through LDS
    ("bf16", 128, 8, 2, 7, (200, 9, 31)),         # 64 rows, one split: output written in place
    ("bf16", 128, 7, 3, 8, (3000, 1500, 17, 260)),  # 63 rows, many splits, odd page counts
    ("f32", 128, 6, 1, 3, (200, 17)),            # 24 rows, fp32
    # gamma = 0: one query per sequence, a plain dense decode step
    ("bf16", 128, 4, 2, 0, (1000, 77, 1)),
    ("f32", 64, 2, 2, 0, (300, 40)),
]


@pytest.mark.parametrize("kv,D,G,Hkv,gamma,ctx", VERIFY_CASES)
def test_dense_verify_matches_oracle(kv, D, G, Hkv, gamma, ctx):
    wl = _make(_cfg(kv, D, G, Hkv, gamma), list(ctx), seed=len(ctx) + D + G)
    scale = 1.0 / np.sqrt(D)
    kvc = _kv(wl, gamma)
    out = s3r.dense_verify_attn(kvc, wl.q_verify, scale)
    torch.cuda.synchronize()
    ref = oracle.dense_verify_attn(f64(wl.q_verify), f64(wl.k_pool), f64(wl.v_pool),
                                   i32(wl.page_table), i32(wl.seq_lens[gamma]), scale)
    _check_attn(out, ref, kv)
    if kv == "bf16":  # bf16 output: the tolerance plus the output's own rounding
        outb = s3r.dense_verify_attn(kvc, wl.q_verify, scale, out_dtype=torch.bfloat16)
        got = outb.float().cpu().numpy()
        assert np.all(np.abs(got - ref) <= 1e-2 + np.abs(ref) * 2.0**-8)


@pytest.mark.parametrize("kv,D", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_page_bounds_exact(kv, D):
    wl = _make(_cfg(kv, D), [300, 17, 48], seed=3)
    kvc = _kv(wl, 0)
    n_phys = wl.k_pool.shape[0]
    bounds = torch.full((n_phys, 2, 2, D), float("nan"), device=DEV).to(wl.k_pool.dtype)
    s3r.page_bounds_update(kvc, bounds)
    torch.cuda.synchronize()
    ref = oracle.page_bounds(f64(wl.k_pool), i32(wl.page_table), i32(wl.seq_lens[0]))
    got = f64(bounds)
    used = ~np.isnan(ref[:, 0, 0, 0])
    assert np.array_equal(got[used], ref[used])
    # Append one token per sequence and refresh only the touched pages.
    kvc1 = _kv(wl, 1)
    first = wl.seq_lens[0].clone()
    s3r.page_bounds_update(kvc1, bounds, first_pos=first, max_pages_touched=1)
    torch.cuda.synchronize()
    ref1 = oracle.page_bounds(f64(wl.k_pool), i32(wl.page_table), i32(wl.seq_lens[1]))
    used1 = ~np.isnan(ref1[:, 0, 0, 0])
    assert np.array_equal(f64(bounds)[used1], ref1[used1])


@pytest.mark.parametrize("kv,D,span", [("bf16", 128, 4), ("f32", 64, 4), ("bf16", 64, 50)])
def test_page_bounds_refresh_over_several_pages(kv, D, span):
    """40 tokens appended past the bounds' length touch four pages (18 to 21
    for L = 300): refreshed from first_pos with max_pages_touched = 4, or a
    larger bound, they equal the oracle's bounds at the new length."""
    wl = _make(_cfg(kv, D, gamma=40), [300, 17, 95], seed=13)
    n_phys = wl.k_pool.shape[0]
    bounds = torch.zeros((n_phys, 2, 2, D), dtype=wl.k_pool.dtype, device=DEV)
    s3r.page_bounds_update(_kv(wl, 0), bounds)
    s3r.page_bounds_update(_kv(wl, 40), bounds, first_pos=wl.seq_lens[0].clone(), max_pages_touched=span)
    torch.cuda.synchronize()
    ref = oracle.page_bounds(f64(wl.k_pool), i32(wl.page_table), i32(wl.seq_lens[40]))
    used = ~np.isnan(ref[:, 0, 0, 0])
    assert np.array_equal(f64(bounds)[used], ref[used])


SELECT_CASES = [
    ("bf16", 128, 4, 2, 64, (700, 300, 40)),
    ("bf16", 128, 2, 2, 160, (2000, 161)),
    ("f32", 64, 2, 2, 64, (512, 513)),
    ("bf16", 64, 8, 1, 32, (999, 1, 16)),
    ("bf16", 128, 3, 2, 64, (700, 31)),
    ("bf16", 64, 7, 1, 48, (400, 200)),
    ("f32", 64, 5, 1, 32, (300, 64)),
    ("bf16", 128, 4, 2, 100, (700, 90, 40)),    # budget not a multiple of P: k = 6
    ("bf16", 64, 2, 2, 16, (500, 17, 1)),       # k = 1
]


@pytest.mark.parametrize("kv,D,G,Hkv,budget,ctx", SELECT_CASES)
def test_page_select_matches_oracle(kv, D, G, Hkv, budget, ctx):
    wl = _make(_cfg(kv, D, G, Hkv, budget=budget, heavy=0), list(ctx), seed=11)
    scale = 1.0 / np.sqrt(D)
    for step in (0, 2):
        kvc = _kv(wl, step)
        bounds = torch.empty((wl.k_pool.shape[0], Hkv, 2, D), dtype=wl.k_pool.dtype, device=DEV)
        s3r.page_bounds_update(kvc, bounds)
        sel, nsel = s3r.page_select(kvc, bounds, wl.draft_q(step), budget, scale)
        torch.cuda.synchronize()
        rb = oracle.page_bounds(f64(wl.k_pool), i32(wl.page_table), i32(wl.seq_lens[step]))
        rsel, rn, rsc = oracle.page_select(rb, f64(wl.draft_q(step)), i32(wl.page_table),
                                           i32(wl.seq_lens[step]), budget, scale)
        check_pages(i32(sel), i32(nsel), rsel, rn, rsc, budget // 16)


DRAFT_CASES = [
    ("bf16", 128, 4, 2, 64, (700, 300, 40)),
    ("bf16", 128, 2, 2, 1024, (3000, 100)),     # many selected pages: several splits
    ("f32", 64, 2, 2, 64, (512, 300)),
    ("bf16", 64, 8, 1, 48, (333, 15)),
    ("bf16", 128, 6, 1, 64, (500, 77)),
    ("bf16", 64, 3, 2, 96, (650, 20)),
]


@pytest.mark.parametrize("kv,D,G,Hkv,budget,ctx", DRAFT_CASES)
def test_sparse_draft_matches_oracle(kv, D, G, Hkv, budget, ctx):
    wl = _make(_cfg(kv, D, G, Hkv, budget=budget), list(ctx), seed=5)
    scale = 1.0 / np.sqrt(D)
    step = 1
    kvc = _kv(wl, step)
    bounds = torch.empty((wl.k_pool.shape[0], Hkv, 2, D), dtype=wl.k_pool.dtype, device=DEV)
    s3r.page_bounds_update(kvc, bounds)
    sel, _ = s3r.page_select(kvc, bounds, wl.draft_q(step), budget, scale)
    out = s3r.sparse_draft_attn(kvc, wl.draft_q(step), sel, scale)
    torch.cuda.synchronize()
    # the oracle attends over the GPU's own selection (selection parity is tested above)
    ref = oracle.sparse_draft_attn(f64(wl.draft_q(step)), f64(wl.k_pool), f64(wl.v_pool),
                                   i32(wl.page_table), i32(wl.seq_lens[step]), i32(sel), scale)
    _check_attn(out, ref, kv)


def test_sparse_draft_handcrafted_selection():
    # -1 holes, unsorted ids and an id past the sequence are all skipped
    wl = _make(_cfg("bf16", 128, 4, 2), [400, 200], seed=9)
    kvc = _kv(wl, 0)
    sel = torch.tensor([[[3, -1, 0, 24, 7], [20, 1, -1, -1, -1]],
                        [[12, 11, 0, 2, 30], [-1, -1, -1, -1, -1]]], dtype=torch.int32, device=DEV)
    out = s3r.sparse_draft_attn(kvc, wl.draft_q(0), sel, 0.1)
    torch.cuda.synchronize()
    n = np.array([oracle.n_pages(x, 16) for x in i32(wl.seq_lens[0])])
    # every entry is read here (k = 5 <= n); ids >= n are skipped like -1
    clean = np.where(i32(sel) < n[:, None, None], i32(sel), -1)
    ref = oracle.sparse_draft_attn(f64(wl.draft_q(0)), f64(wl.k_pool), f64(wl.v_pool),
                                   i32(wl.page_table), i32(wl.seq_lens[0]), clean, 0.1)
    got = out.cpu().numpy()
    assert np.all(got[1, 4:] == 0)            # an empty selection row gives zeros
    ok = ~np.isnan(ref)
    assert np.max(np.abs(got[ok] - ref[ok])) <= 1e-2


def _sample_case(B, gamma, V, noise, seed, T=1.0):
    g = torch.Generator().manual_seed(seed)
    d = torch.randn((B, gamma, V), generator=g) * 2.0
    t = torch.cat([d + torch.randn((B, gamma, V), generator=g) * noise,
                   torch.randn((B, 1, V), generator=g) * 2.0], dim=1)
    x = oracle.draw_draft_tokens(d.double().numpy(), T, seed=seed, offset=0)
    return d, t, torch.from_numpy(x)


@pytest.mark.parametrize("B,gamma,V,noise,T", [
    (64, 4, 1024, 0.5, 1.0), (16, 6, 151936, 0.5, 1.0), (24, 8, 32000, 1.35, 1.0),
    (32, 2, 5000, 3.0, 1.0), (8, 3, 4099, 0.7, 0.6), (40, 1, 100, 0.0, 1.0),
    (4, 16, 2001, 0.5, 1.0),   # the longest draft the library takes
    (8, 3, 1, 0.5, 1.0),       # one-token vocabulary: p = q = 1, every draft accepted
    (16, 1, 2, 1.0, 1.0)])     # two tokens, one draft
def test_spec_sample_matches_oracle(B, gamma, V, noise, T):
    d, t, x = _sample_case(B, gamma, V, noise, seed=B + V, T=T)
    out, n = s3r.spec_sample(d.to(DEV), t.to(DEV), x.to(DEV).int(), T, seed=0, offset=7)
    torch.cuda.synchronize()
    ro, rn, dec = oracle.spec_sample(d.double().numpy(), t.double().numpy(), x.numpy(), T, 0, 7)
    full = check_tokens(i32(out), i32(n), ro, rn, dec)
    assert full >= B // 2, (full, B)
    if noise == 0.0 or V == 1:
        assert np.all(i32(n) == gamma)
    if V == 1:
        assert np.all(i32(out) == 0)


@pytest.mark.parametrize("B,gamma,V,T", [(16, 4, 32000, 0.8), (8, 6, 151936, 1.0)])
def test_spec_sample_masked_logits(B, gamma, V, T):
    """Masked vocabularies (-inf logits): random masks in both distributions, so
    many drafts have p(x) = 0, and a masked vocabulary tail that fills whole
    4096-token chunks (their statistics are empty). Every emitted token must
    have p > 0 at its slot, and the tokens follow the oracle."""
    g = torch.Generator().manual_seed(V + B)
    d = torch.randn((B, gamma, V), generator=g) * 2.0
    t = torch.cat([d + torch.randn((B, gamma, V), generator=g) * 0.7,
                   torch.randn((B, 1, V), generator=g) * 2.0], dim=1)
    d[torch.rand(d.shape, generator=g) < 0.5] = float("-inf")
    t[torch.rand(t.shape, generator=g) < 0.3] = float("-inf")
    tail = V - V // 3
    d[..., tail:] = float("-inf")
    t[..., tail:] = float("-inf")
    x = oracle.draw_draft_tokens(d.double().numpy(), T, seed=V, offset=0)
    out, n = s3r.spec_sample(d.to(DEV), t.to(DEV), torch.from_numpy(x).to(DEV).int(), T, seed=3, offset=1)
    torch.cuda.synchronize()
    ro, rn, dec = oracle.spec_sample(d.double().numpy(), t.double().numpy(), x, T, 3, 1)
    full = check_tokens(i32(out), i32(n), ro, rn, dec)
    assert full >= B // 2, (full, B)
    go, gn = i32(out), i32(n)
    for b in range(B):
        for i in range(gn[b] + 1):
            assert np.isfinite(t[b, i, go[b, i]].item()), (b, i, go[b, i])
    assert np.any(gn < gamma)  # the masks make rejections happen


def test_spec_sample_masked_leading_passes():
    """A vocabulary of more than 128 chunks of 4096 tokens whose first 2 * 64
    chunks are masked in every row: the row statistics fold two passes of 64
    chunks without mass before the first pass with mass. The tokens follow
    the oracle and lie in the unmasked tail."""
    B, gamma, V, T = 4, 3, 600000, 1.0
    masked = 2 * 64 * 4096
    d, t, _ = _sample_case(B, gamma, V, 0.7, seed=77)
    d[..., :masked] = float("-inf")
    t[..., :masked] = float("-inf")
    x = oracle.draw_draft_tokens(d.double().numpy(), T, seed=5, offset=0)
    out, n = s3r.spec_sample(d.to(DEV), t.to(DEV), torch.from_numpy(x).to(DEV).int(), T, seed=2, offset=0)
    torch.cuda.synchronize()
    ro, rn, dec = oracle.spec_sample(d.double().numpy(), t.double().numpy(), x, T, 2, 0)
    full = check_tokens(i32(out), i32(n), ro, rn, dec)
    assert full >= B // 2, (full, B)
    go, gn = i32(out), i32(n)
    for b in range(B):
        assert np.all(go[b, :gn[b] + 1] >= masked) and np.all(go[b, gn[b] + 1:] == -1), b


def test_determinism_bitwise():
    wl = _make(_cfg("bf16", 128, 4, 2, 6), [900, 300], seed=21)
    kvc = _kv(wl, 6)
    a = s3r.dense_verify_attn(kvc, wl.q_verify, 0.09)
    b = s3r.dense_verify_attn(kvc, wl.q_verify, 0.09)
    d, t, x = _sample_case(8, 4, 20000, 0.5, seed=3)
    o1 = s3r.spec_sample(d.to(DEV), t.to(DEV), x.to(DEV).int(), 1.0, 1, 2)
    o2 = s3r.spec_sample(d.to(DEV), t.to(DEV), x.to(DEV).int(), 1.0, 1, 2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(o1[0], o2[0]) and torch.equal(o1[1], o2[1])
    # a different Philox offset gives a different stream
    o3 = s3r.spec_sample(d.to(DEV), t.to(DEV), x.to(DEV).int(), 1.0, 1, 3)
    assert not torch.equal(o1[0], o3[0]) or not torch.equal(o1[1], o3[1])


@pytest.mark.parametrize("G,gamma", [(4, 6), (4, 8), (8, 7)], ids=["rows28", "rows36", "rows64"])
def test_split_count_invariance(G, gamma):
    """The page hint changes the split plan (register, K-ring and LDS-staged
    pipelines alike), not the result."""
    wl = _make(_cfg("bf16", 128, G, 2, gamma), [1500, 700], seed=22)
    outs = []
    for hint in (0, 200, 60):
        kvc = _kv(wl, gamma, hint=hint)
        outs.append(s3r.dense_verify_attn(kvc, wl.q_verify, 0.09).cpu())
    for o in outs[1:]:
        assert torch.max(torch.abs(o - outs[0])) <= 1e-5


def test_unselected_pages_do_not_affect_draft():
    wl = _make(_cfg("bf16", 128, 4, 2, 4, budget=64), [600, 450], seed=23)
    kvc = _kv(wl, 0)
    bounds = torch.empty((wl.k_pool.shape[0], 2, 2, 128), dtype=torch.bfloat16, device=DEV)
    s3r.page_bounds_update(kvc, bounds)
    sel, _ = s3r.page_select(kvc, bounds, wl.draft_q(0), 64, 0.09)
    d0 = s3r.sparse_draft_attn(kvc, wl.draft_q(0), sel, 0.09).clone()
    v0 = s3r.dense_verify_attn(kvc, wl.q_verify[:, :1].contiguous(), 0.09).clone()
    # perturb every page no (sequence, kv head) selected
    keep = set()
    pt = wl.page_table.cpu()
    for b in range(2):
        for j in sel[b].flatten().tolist():
            if j >= 0:
                keep.add(int(pt[b, j]))
    mask = torch.ones(wl.k_pool.shape[0], dtype=torch.bool)
    mask[list(keep)] = False
    idx = mask.nonzero().flatten().to(DEV)
    wl.v_pool[idx] = (wl.v_pool[idx].float() + 1.0).to(torch.bfloat16)
    d1 = s3r.sparse_draft_attn(kvc, wl.draft_q(0), sel, 0.09)
    v1 = s3r.dense_verify_attn(kvc, wl.q_verify[:, :1].contiguous(), 0.09)
    torch.cuda.synchronize()
    assert torch.equal(d0, d1)
    assert not torch.equal(v0, v1)


def test_verify_row_equals_draft_over_all_pages():
    gamma = 4
    wl = _make(_cfg("bf16", 128, 4, 2, gamma, budget=4096), [555, 301], seed=24)
    kvv = _kv(wl, gamma)
    ver = s3r.dense_verify_attn(kvv, wl.q_verify, 0.09)
    for i in range(gamma + 1):
        kvd = _kv(wl, i)  # seq_len = S - gamma + i
        sel = torch.arange(256, dtype=torch.int32, device=DEV).repeat(2, 2, 1).contiguous()
        dr = s3r.sparse_draft_attn(kvd, wl.draft_q(i), sel, 0.09)
        torch.cuda.synchronize()
        assert torch.max(torch.abs(dr - ver[:, i])) <= 1e-5


@pytest.mark.parametrize("G,gamma", [(4, 4), (4, 8), (8, 7)], ids=["rows20", "rows36", "rows64"])
def test_edge_cases_empty_and_short(G, gamma):
    """An empty sequence, one shorter than the verify queries and a single
    page, through the register (20 rows), K-ring (36) and LDS-staged (64)
    verify pipelines."""
    wl = _make(_cfg("bf16", 128, G, 2, gamma), [40, 3, 1], seed=25)
    seq = torch.tensor([0, 3, 16], dtype=torch.int32, device=DEV)  # empty, shorter than n_q, one page
    kvc = s3r.PagedKVCache(wl.k_pool, wl.v_pool, wl.page_table, seq, wl.cfg["Hq"])
    out = s3r.dense_verify_attn(kvc, wl.q_verify, 0.1)
    torch.cuda.synchronize()
    ref = oracle.dense_verify_attn(f64(wl.q_verify), f64(wl.k_pool), f64(wl.v_pool),
                                   i32(wl.page_table), seq.cpu().numpy(), 0.1)
    assert np.all(out[0].cpu().numpy() == 0)
    assert np.all(out[1, :2].cpu().numpy() == 0)
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= 1e-2
    bounds = torch.zeros((wl.k_pool.shape[0], 2, 2, 128), dtype=torch.bfloat16, device=DEV)
    s3r.page_bounds_update(kvc, bounds)
    sel, n = s3r.page_select(kvc, bounds, wl.draft_q(0), 32, 0.1)
    torch.cuda.synchronize()
    assert i32(n).tolist() == [0, 1, 1]
    assert i32(sel)[0].tolist() == [[-1, -1], [-1, -1]]
    assert i32(sel)[1].tolist() == [[0, -1], [0, -1]]
    dr = s3r.sparse_draft_attn(kvc, wl.draft_q(0), sel, 0.1)
    torch.cuda.synchronize()
    assert np.all(dr[0].cpu().numpy() == 0)


FUSED_CASES = [
    ("bf16", 128, 4, 2, 64, (700, 300, 40)),
    ("bf16", 128, 2, 2, 1024, (3000, 100)),    # selection longer than one workgroup's splits
    ("bf16", 64, 8, 1, 48, (333, 15)),
    ("bf16", 128, 4, 2, 4096, (100, 50)),      # budget covers every page
    ("bf16", 128, 4, 2, 320000, (900, 30)),    # k = 20000: the list no longer fits LDS, three launches
    ("bf16", 64, 4, 2, 64, (8000, 7990)),      # 4 pages of 500, eight waves
    ("bf16", 128, 4, 2, 64, (9000, 200)),      # 4 pages of 563
    ("bf16", 64, 2, 1, 64, (140000, 300)),     # 8750 pages: past the fused top-k
    # 32 sequences x 8 kv heads fill the device: the single-kernel step (scores
    # in LDS); ragged lengths, some short enough that every page is taken
    ("bf16", 128, 4, 8, 512, tuple(60 + 97 * i for i in range(32))),
    ("bf16", 64, 8, 8, 256, tuple(3000 - 90 * i for i in range(32))),
    ("bf16", 128, 1, 8, 2048, tuple(2100 + 61 * i for i in range(32))),
    ("bf16", 128, 4, 8, 1000, tuple(900 + 53 * i for i in range(32))),  # k = 62 over eight waves
    ("bf16", 128, 4, 8, 16, tuple(300 + 7 * i for i in range(32))),    # k = 1: one wave attends
    ("f32", 64, 2, 2, 64, (512, 300)),         # fp32: the separate kernels
    # groups that are not a power of two take the score kernel + attention
    ("bf16", 128, 3, 2, 64, (700, 300)),
    ("bf16", 64, 5, 2, 48, (1000, 20)),
    ("bf16", 128, 6, 8, 512, tuple(60 + 97 * i for i in range(32))),  # fills the device
    ("bf16", 64, 7, 1, 64, (9000, 150)),
    # 64 sequences x 8 kv heads: two (sequence, kv head) pairs per CU, so the
    # single-kernel step runs four-wave workgroups, two per CU
    ("bf16", 128, 2, 8, 256, tuple(50 + 37 * i for i in range(64))),
    ("bf16", 64, 8, 8, 128, tuple(900 - 13 * i for i in range(64))),
    # ... one outlier past 2048 pages: at four waves its workgroups would end the
    # kernel long after the rest, so the step runs eight (the four-wave, 32-key
    # top-k needs a balanced batch of long tables: test_fullsize_ragged[128])
    ("bf16", 128, 2, 8, 256, (40000,) + tuple(100 + 7 * i for i in range(63))),
    # 2048 (sequence, kv head) pairs with k = 8750: eight waves' window tables
    # would pass 64 KB of LDS, so the draft keeps the attention's own plan
    ("bf16", 64, 2, 8, 140000, tuple(300 + 13 * (i % 7) for i in range(256))),
]


@pytest.mark.parametrize("kv,D,G,Hkv,budget,ctx", FUSED_CASES)
def test_fused_draft_step_equals_separate_calls(kv, D, G, Hkv, budget, ctx):
    wl = _make(_cfg(kv, D, G, Hkv, budget=budget), list(ctx), seed=31)
    scale = 1.0 / np.sqrt(D)
    gamma = wl.cfg["gamma"]
    # bounds as of the whole pre-filled KV: the step's tail page is stale until refreshed
    stale = torch.empty((wl.k_pool.shape[0], Hkv, 2, D), dtype=wl.k_pool.dtype, device=DEV)
    s3r.page_bounds_update(_kv(wl, gamma), stale)
    for step in (0, 1, 3):
        kvc = _kv(wl, step)
        first = (wl.seq_lens[step] - 1).contiguous()
        q = wl.draft_q(step)
        ba = stale.clone()
        s3r.page_bounds_update(kvc, ba, first_pos=first, max_pages_touched=1)
        sel_a, n_a = s3r.page_select(kvc, ba, q, budget, scale)
        out_a = s3r.sparse_draft_attn(kvc, q, sel_a, scale)
        bb = stale.clone()
        out_b, sel_b, n_b = s3r.sparse_draft_step(kvc, bb, q, budget, scale, refresh_from=first)
        torch.cuda.synchronize()
        assert torch.equal(ba, bb)
        assert torch.equal(sel_a, sel_b) and torch.equal(n_a, n_b)
        # the same pages and arithmetic; only the split-KV merge order may differ
        torch.testing.assert_close(out_b, out_a, rtol=1e-5, atol=1e-5)
        # and against the oracle: bounds, selection (tie window) and attention
        L = i32(wl.seq_lens[step])
        rb = oracle.page_bounds(f64(wl.k_pool), i32(wl.page_table), L)
        used = ~np.isnan(rb[:, 0, 0, 0])
        assert np.array_equal(f64(bb)[used], rb[used])
        rsel, rn, rsc = oracle.page_select(rb, f64(q), i32(wl.page_table), L, budget, scale)
        check_pages(i32(sel_b), i32(n_b), rsel, rn, rsc, budget // 16)
        ref = oracle.sparse_draft_attn(f64(q), f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table),
                                       L, i32(sel_b), scale)
        _check_attn(out_b, ref, kv)


def _check_round_pages(sel, nsel, rsel, rn, rsc, L, gamma, k, max_pages, tie=1e-4):
    """Forced pages exactly; the scored rest within the tie window of the oracle's."""
    assert np.array_equal(nsel, rn), (nsel, rn)
    for b in range(sel.shape[0]):
        forced = oracle.round_forced_pages(int(L[b]), gamma, 16, max_pages)
        for h in range(sel.shape[1]):
            g = [int(x) for x in sel[b, h] if x >= 0]
            r = [int(x) for x in rsel[b, h] if x >= 0]
            assert g == sorted(g) and len(g) == len(r), (b, h, g, r)
            assert set(forced) <= set(g), (b, h, forced, g)
            if g == r:
                continue
            sc = rsc[(b, h)]
            kth = sorted(sc.values(), reverse=True)[k - len(forced) - 1]
            for j in set(g) ^ set(r):
                assert j in sc and abs(sc[j] - kth) <= tie, (b, h, j, kth)


ROUND_CASES = [
    # kv, D, G, Hkv, budget, gamma, ctx
    ("bf16", 128, 4, 8, 512, 6, tuple(60 + 97 * i for i in range(32))),  # one kernel
    ("bf16", 128, 4, 2, 64, 4, (700, 300, 47, 31)),   # two kernels; rounds that open a page
    ("bf16", 64, 2, 2, 48, 16, (333, 15, 32)),        # gamma 16, short sequences
    ("f32", 64, 2, 2, 64, 3, (512, 300, 64)),         # fp32: the separate kernels
    ("bf16", 128, 4, 2, 64, 2, (9000, 200)),          # 563 pages, two kernels
    ("bf16", 64, 2, 1, 64, 5, (140000, 300)),         # 8750 pages: past the fused top-k
    ("bf16", 128, 3, 2, 64, 4, (700, 300, 47)),       # G = 3: score kernel + attention
    ("bf16", 64, 6, 8, 256, 6, tuple(90 + 61 * i for i in range(32))),  # G = 6, device-filling
    ("bf16", 128, 2, 8, 256, 4, tuple(40 + 29 * i for i in range(64))),  # four-wave single kernel
    ("bf16", 64, 4, 8, 128, 3, (30000,) + tuple(60 + 11 * i for i in range(63))),  # one outlier: eight waves
]


@pytest.mark.parametrize("kv,D,G,Hkv,budget,gamma,ctx", ROUND_CASES)
def test_round_selection_then_reuse(kv, D, G, Hkv, budget, gamma, ctx):
    wl = _make(_cfg(kv, D, G, Hkv, gamma=gamma, budget=budget), list(ctx), seed=41)
    scale = 1.0 / np.sqrt(D)
    bounds = torch.empty((wl.k_pool.shape[0], Hkv, 2, D), dtype=wl.k_pool.dtype, device=DEV)
    s3r.page_bounds_update(_kv(wl, gamma), bounds)  # stale tail pages until refreshed
    first = (wl.seq_lens[0] - 1).contiguous()
    out0, sel, nsel = s3r.sparse_draft_round(_kv(wl, 0), bounds, wl.draft_q(0), budget, gamma,
                                             scale, refresh_from=first)
    torch.cuda.synchronize()
    L0 = i32(wl.seq_lens[0])
    pt = i32(wl.page_table)
    rb = oracle.page_bounds(f64(wl.k_pool), pt, L0)
    used = ~np.isnan(rb[:, 0, 0, 0])
    assert np.array_equal(f64(bounds)[used], rb[used])
    rsel, rn, rsc = oracle.page_select_round(rb, f64(wl.draft_q(0)), pt, L0, budget, gamma, scale)
    _check_round_pages(i32(sel), i32(nsel), rsel, rn, rsc, L0, gamma, budget // 16, pt.shape[1])
    K, V = f64(wl.k_pool), f64(wl.v_pool)
    ref = oracle.sparse_draft_attn(f64(wl.draft_q(0)), K, V, pt, L0, i32(sel), scale)
    _check_attn(out0, ref, kv)
    for j in range(1, gamma):  # the round's later steps reuse the selection
        out = s3r.sparse_draft_attn(_kv(wl, j), wl.draft_q(j), sel, scale)
        torch.cuda.synchronize()
        ref = oracle.sparse_draft_attn(f64(wl.draft_q(j)), K, V, pt, i32(wl.seq_lens[j]), i32(sel),
                                       scale)
        _check_attn(out, ref, kv)


COMMIT_CASES = [
    # kv, D, Hkv, ctx, count, table slack (gamma), accepted per sequence
    ("bf16", 128, 2, (40, 17, 64, 100), 7, 8, (6, 0, 2, 7)),
    ("f32", 64, 2, (15, 16, 200), 3, 4, (2, 2, 0)),
    ("bf16", 64, 3, (33, 1), 1, 2, (0, 1)),
    ("bf16", 128, 2, (60,), 8, 2, (4,)),          # rows past the table are dropped
    ("bf16", 128, 2, (45, 70), 0, 2, (-10, -3)),  # a pure rollback
]


@pytest.mark.parametrize("kv,D,Hkv,ctx,count,slack,accepted", COMMIT_CASES)
def test_kv_commit_matches_oracle(kv, D, Hkv, ctx, count, slack, accepted):
    wl = _make(_cfg(kv, D, 2, Hkv, gamma=slack), list(ctx), seed=51)
    dt = wl.k_pool.dtype
    bounds = torch.empty((wl.k_pool.shape[0], Hkv, 2, D), dtype=dt, device=DEV)
    s3r.page_bounds_update(_kv(wl, 0), bounds)
    first = (wl.seq_lens[0] - 1).contiguous()
    committed = (first + 1 + torch.tensor(accepted, dtype=torch.int32, device=DEV)).contiguous()
    g = torch.Generator(device="cpu").manual_seed(52)
    k_new = torch.randn((len(ctx), count, Hkv, D), generator=g).to(dt).to(DEV)
    v_new = torch.randn((len(ctx), count, Hkv, D), generator=g).to(dt).to(DEV)
    K0, V0, B0 = f64(wl.k_pool), f64(wl.v_pool), f64(bounds)
    rK, rV, rB = oracle.kv_commit(K0, V0, i32(wl.page_table), f64(k_new), f64(v_new), i32(first),
                                  i32(committed), B0)
    kvc = s3r.PagedKVCache(wl.k_pool, wl.v_pool, wl.page_table, committed, wl.cfg["Hq"])
    s3r.kv_commit(kvc, k_new, v_new, first, bounds)
    torch.cuda.synchronize()
    assert np.array_equal(f64(wl.k_pool), rK)
    assert np.array_equal(f64(wl.v_pool), rV)
    assert np.array_equal(f64(bounds), rB, equal_nan=True)


@pytest.mark.parametrize("G,gamma", [(4, 4), (4, 8), (8, 7)], ids=["rows20", "rows36", "rows64"])
def test_ragged_longest_first_matches_oracle(G, gamma):
    """A ragged batch with its page hint set: the attention workgroups take the
    sequences longest first (verify and the draft step), with the finer splits
    of a batch of few pairs; 36 and 64 verify rows run the K-ring and the
    LDS-staged pipelines."""
    ctx = (5000, 40, 700, 17, 2300, 64)
    budget = 256
    wl = _make(_cfg("bf16", 128, G, 2, gamma=gamma, budget=budget), list(ctx), seed=61)
    total = sum(-(-(L + gamma) // 16) for L in ctx)
    assert wl.max_pages * len(ctx) > 2 * total  # ragged enough to reorder
    scale = 1.0 / np.sqrt(128)
    K, V, pt = f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table)
    out = s3r.dense_verify_attn(_kv(wl, gamma, hint=total), wl.q_verify, scale)
    torch.cuda.synchronize()
    ref = oracle.dense_verify_attn(f64(wl.q_verify), K, V, pt, i32(wl.seq_lens[gamma]), scale)
    _check_attn(out, ref, "bf16")
    bounds = torch.empty((wl.k_pool.shape[0], 2, 2, 128), dtype=wl.k_pool.dtype, device=DEV)
    s3r.page_bounds_update(_kv(wl, 0), bounds)
    kv0 = _kv(wl, 0, hint=total)
    q0 = wl.draft_q(0)
    d_out, sel, nsel = s3r.sparse_draft_step(kv0, bounds, q0, budget, scale,
                                             refresh_from=(wl.seq_lens[0] - 1).contiguous())
    torch.cuda.synchronize()
    L0 = i32(wl.seq_lens[0])
    rb = oracle.page_bounds(K, pt, L0)
    rsel, rn, rsc = oracle.page_select(rb, f64(q0), pt, L0, budget, scale)
    check_pages(i32(sel), i32(nsel), rsel, rn, rsc, budget // 16)
    ref = oracle.sparse_draft_attn(f64(q0), K, V, pt, L0, i32(sel), scale)
    _check_attn(d_out, ref, "bf16")


def test_longest_first_many_sequences_with_ties():
    """1300 sequences (two 1024-length LDS passes of the ordering, six blocks),
    most lengths shared, one long: every sequence must be taken exactly once.
    Outputs start as NaN so a sequence the order skips cannot pass."""
    rng = np.random.default_rng(71)
    ctx = [int(x) for x in rng.choice([20, 33, 64, 150], size=1300)]
    ctx[700] = 3000
    gamma, budget = 2, 64
    wl = _make(_cfg("bf16", 64, 2, 1, gamma=gamma, budget=budget), ctx, seed=71)
    total = sum(-(-(L + gamma) // 16) for L in ctx)
    assert wl.max_pages * len(ctx) > 2 * total
    scale = 0.125
    K, V, pt = f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table)
    out = torch.full((len(ctx), gamma + 1, 2, 64), float("nan"), device=DEV)
    s3r.dense_verify_attn(_kv(wl, gamma, hint=total), wl.q_verify, scale, out=out)
    bounds = torch.empty((wl.k_pool.shape[0], 1, 2, 64), dtype=wl.k_pool.dtype, device=DEV)
    s3r.page_bounds_update(_kv(wl, 0), bounds)
    q0 = wl.draft_q(0)
    d_out = torch.full((len(ctx), 2, 64), float("nan"), device=DEV)
    _, sel, nsel = s3r.sparse_draft_step(_kv(wl, 0, hint=total), bounds, q0, budget, scale,
                                         refresh_from=(wl.seq_lens[0] - 1).contiguous(), out=d_out)
    torch.cuda.synchronize()
    ref = oracle.dense_verify_attn(f64(wl.q_verify), K, V, pt, i32(wl.seq_lens[gamma]), scale)
    _check_attn(out, ref, "bf16")
    L0 = i32(wl.seq_lens[0])
    rsel, rn, rsc = oracle.page_select(oracle.page_bounds(K, pt, L0), f64(q0), pt, L0, budget, scale)
    check_pages(i32(sel), i32(nsel), rsel, rn, rsc, budget // 16)
    _check_attn(d_out, oracle.sparse_draft_attn(f64(q0), K, V, pt, L0, i32(sel), scale), "bf16")


@pytest.mark.parametrize("hint", [False, True], ids=["plain", "ragged_hint"])
def test_very_long_context(hint):
    """300K tokens (18753 pages) beside a 50-token sequence: verify over many
    split groups and the global combine, and a sparse draft over 64 pages
    spread across the whole context (past what the in-kernel top-k ranks)."""
    ctx = [300000, 50]
    gamma = 3
    wl = _make(_cfg("bf16", 64, 2, 1, gamma=gamma, budget=1024), ctx, seed=81)
    total = sum(-(-(L + gamma) // 16) for L in ctx) if hint else 0
    K, V, pt = f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table)
    out = s3r.dense_verify_attn(_kv(wl, gamma, hint=total), wl.q_verify, 0.125)
    rng = np.random.default_rng(81)
    sel = np.full((2, 1, 64), -1, dtype=np.int32)
    sel[0, 0] = np.sort(rng.choice(18750, size=64, replace=False))
    sel[1, 0, :4] = np.arange(4)
    d_out = s3r.sparse_draft_attn(_kv(wl, 0, hint=total), wl.draft_q(0), torch.from_numpy(sel).to(DEV),
                                  0.125)
    torch.cuda.synchronize()
    ref = oracle.dense_verify_attn(f64(wl.q_verify), K, V, pt, i32(wl.seq_lens[gamma]), 0.125)
    _check_attn(out, ref, "bf16")
    rd = oracle.sparse_draft_attn(f64(wl.draft_q(0)), K, V, pt, i32(wl.seq_lens[0]), sel, 0.125)
    _check_attn(d_out, rd, "bf16")


def test_k_ring_verify_at_scale():
    """36 verify rows over 512 (sequence, kv head) pairs of 40000 tokens (10 GB of
    KV): the K-ring pipeline with splits long enough that the plan caps each
    wave's window table at 1024 pages. Checked on every kv head of the first
    and last sequences and on a seeded sample of the rest."""
    gamma = 8
    wl = make_workload("qwen3_8b", device=DEV, seed=5, with_logits=False, B=64, L=40000, gamma=gamma)
    cfg = wl.cfg
    B, Hq, Hkv, D, P = (cfg[k] for k in ("B", "Hq", "Hkv", "D", "P"))
    assert (Hq // Hkv) * (gamma + 1) == 36
    total = sum(-(-(int(L) + gamma) // P) for L in wl.ctx)
    kv = s3r.PagedKVCache(wl.k_pool, wl.v_pool, wl.page_table, wl.seq_lens[gamma], Hq, total_pages_hint=total)
    scale = 1.0 / np.sqrt(D)
    out = s3r.dense_verify_attn(kv, wl.q_verify, scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    slices = sorted({(0, h) for h in range(Hkv)} | {(B - 1, h) for h in range(Hkv)} |
                    {(int(b), int(h)) for b, h in zip(rng.integers(0, B, 4), rng.integers(0, Hkv, 4))})
    G = Hq // Hkv
    for b, h in slices:
        n = -(-(int(wl.ctx[b]) + gamma) // P)
        idx = wl.page_table[b, :n].long()
        K = wl.k_pool.index_select(0, idx)[:, h:h + 1].to("cpu", torch.float64).numpy()
        V = wl.v_pool.index_select(0, idx)[:, h:h + 1].to("cpu", torch.float64).numpy()
        q = wl.q_verify[b:b + 1, :, h * G:(h + 1) * G].to("cpu", torch.float64).numpy()
        ref = oracle.dense_verify_attn(q, K, V, np.arange(n, dtype=np.int64)[None, :],
                                       np.array([int(wl.seq_lens[gamma][b])], dtype=np.int32), scale)
        print(f"k-ring at scale: slice ({b}, {h})", flush=True)
        _check_attn(out[b:b + 1, :, h * G:(h + 1) * G], ref, "bf16")


def test_round_and_commit_edge_cases():
    """Empty, one-token and page-boundary lengths through the once-per-round
    selection (k = 2 pages, gamma = 3) and a 3-row KV commit."""
    gamma, budget = 3, 32
    wl = _make(_cfg("bf16", 128, 4, 2, gamma=gamma, budget=budget), [8, 8, 20, 20, 20, 40], seed=27)
    seq = torch.tensor([0, 1, 15, 16, 17, 33], dtype=torch.int32, device=DEV)
    kvc = s3r.PagedKVCache(wl.k_pool, wl.v_pool, wl.page_table, seq, wl.cfg["Hq"])
    bounds = torch.zeros((wl.k_pool.shape[0], 2, 2, 128), dtype=torch.bfloat16, device=DEV)
    s3r.page_bounds_update(kvc, bounds)
    q0 = wl.draft_q(0)
    out, sel, nsel = s3r.sparse_draft_round(kvc, bounds, q0, budget, gamma, 0.1)
    torch.cuda.synchronize()
    K, V, pt, L = f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table), i32(seq)
    rb = oracle.page_bounds(K, pt, L)
    rsel, rn, _ = oracle.page_select_round(rb, f64(q0), pt, L, budget, gamma, 0.1)
    assert np.array_equal(i32(sel), rsel) and np.array_equal(i32(nsel), rn), (i32(sel), rsel)
    assert i32(sel)[0].tolist() == [[0, -1], [0, -1]]  # nothing yet: the round's first page
    ref = oracle.sparse_draft_attn(f64(q0), K, V, pt, L, rsel, 0.1)
    assert np.all(out[0].cpu().numpy() == 0)
    _check_attn(out, ref, "bf16")
    first = torch.clamp(seq - 1, min=0).contiguous()
    committed = (first + torch.tensor([1, 0, 2, 3, 1, 2], dtype=torch.int32, device=DEV)).contiguous()
    g = torch.Generator(device="cpu").manual_seed(28)
    k_new = torch.randn((6, 3, 2, 128), generator=g).to(torch.bfloat16).to(DEV)
    v_new = torch.randn((6, 3, 2, 128), generator=g).to(torch.bfloat16).to(DEV)
    B0 = f64(bounds)
    rK, rV, rB = oracle.kv_commit(K, V, pt, f64(k_new), f64(v_new), i32(first), i32(committed), B0)
    kvc.set_seq_lens(committed)
    s3r.kv_commit(kvc, k_new, v_new, first, bounds)
    torch.cuda.synchronize()
    assert np.array_equal(f64(wl.k_pool), rK) and np.array_equal(f64(wl.v_pool), rV)
    assert np.array_equal(f64(bounds), rB)


def test_select_at_the_page_limit():
    """page_select and the draft step at the select kernel's 32768-page limit
    (the draft step's fused paths stop at 8192 and hand over to the separate
    kernels), and a table one page wider, refused before any launch."""
    gamma, budget = 4, 256
    ctx = 32768 * 16 - gamma  # the table holds ctx + gamma positions: 32768 pages
    wl = _make(_cfg("bf16", 64, 2, 1, gamma=gamma, budget=budget), [ctx], seed=71)
    assert wl.max_pages == 32768
    kvc = _kv(wl, 0)
    bounds = torch.empty((wl.k_pool.shape[0], 1, 2, 64), dtype=wl.k_pool.dtype, device=DEV)
    s3r.page_bounds_update(kvc, bounds)
    q0 = wl.draft_q(0)
    sel, nsel = s3r.page_select(kvc, bounds, q0, budget, 0.125)
    out, sel2, nsel2 = s3r.sparse_draft_step(kvc, bounds, q0, budget, 0.125,
                                            refresh_from=(wl.seq_lens[0] - 1).contiguous())
    torch.cuda.synchronize()
    K, V, pt, L = f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table), i32(wl.seq_lens[0])
    rb = oracle.page_bounds(K, pt, L)
    rsel, rn, rsc = oracle.page_select(rb, f64(q0), pt, L, budget, 0.125)
    check_pages(i32(sel), i32(nsel), rsel, rn, rsc, budget // 16)
    assert torch.equal(sel, sel2) and torch.equal(nsel, nsel2)
    ref = oracle.sparse_draft_attn(f64(q0), K, V, pt, L, i32(sel2), 0.125)
    _check_attn(out, ref, "bf16")
    wide = torch.zeros((1, 32769), dtype=torch.int32, device=DEV)
    big = s3r.PagedKVCache(wl.k_pool, wl.v_pool, wide, wl.seq_lens[0], wl.cfg["Hq"])
    with pytest.raises(s3r.S3RError):
        s3r.page_select(big, bounds, q0, budget, 0.125)
    with pytest.raises(s3r.S3RError):
        s3r.sparse_draft_step(big, bounds, q0, budget, 0.125)


def test_kv_commit_skips_unallocated_pages():
    """Rows aimed at a page whose table entry is -1 are dropped on both sides."""
    wl = _make(_cfg("bf16", 64, 2, 2, gamma=6), [30, 45], seed=53)
    pt = wl.page_table.clone()
    pt[0, 2] = -1
    pt[1, 3] = -1
    bounds = torch.zeros((wl.k_pool.shape[0], 2, 2, 64), dtype=torch.bfloat16, device=DEV)
    first = (wl.seq_lens[0] - 1).contiguous()
    committed = (first + 4).contiguous()
    g = torch.Generator(device="cpu").manual_seed(54)
    k_new = torch.randn((2, 5, 2, 64), generator=g).to(torch.bfloat16).to(DEV)
    v_new = torch.randn((2, 5, 2, 64), generator=g).to(torch.bfloat16).to(DEV)
    rK, rV, rB = oracle.kv_commit(f64(wl.k_pool), f64(wl.v_pool), i32(pt), f64(k_new), f64(v_new),
                                  i32(first), i32(committed), f64(bounds))
    kvc = s3r.PagedKVCache(wl.k_pool, wl.v_pool, pt, committed, wl.cfg["Hq"])
    s3r.kv_commit(kvc, k_new, v_new, first, bounds)
    torch.cuda.synchronize()
    assert np.array_equal(f64(wl.k_pool), rK) and np.array_equal(f64(wl.v_pool), rV)
    assert np.array_equal(f64(bounds), rB)


# Small budgets over long tables (the aggressive shape's k = 16 of 4097
# pages), tables within the budget, and every score tied (the lowest pages
# must win), through page_select and the draft step.
CANDIDATE_CASES = [
    # kv, D, G, Hkv, budget, ctx, constant keys (every score ties)
    ("bf16", 128, 4, 2, 256, (65536, 4000, 130), False),  # 4097, 251 and 9 pages, k = 16
    ("bf16", 128, 4, 2, 1024, (40000, 16000), False),     # k = 64 of 2501 / 1001 pages
    ("bf16", 64, 2, 1, 256, (8000,), True),               # 500 tied pages
    ("bf16", 64, 2, 1, 256, (20000,), True),              # 1250 tied pages
    ("f32", 64, 2, 2, 128, (9000, 3000), False),          # fp32 scores through the separate top-k
]


@pytest.mark.parametrize("kv,D,G,Hkv,budget,ctx,tied", CANDIDATE_CASES)
def test_small_budget_ranking_matches_oracle(kv, D, G, Hkv, budget, ctx, tied):
    wl = _make(_cfg(kv, D, G, Hkv, budget=budget), list(ctx), seed=23)
    if tied:
        wl.k_pool.fill_(0.5)
    scale = 1.0 / np.sqrt(D)
    k = budget // 16
    for step in (0, 3):
        kvc = _kv(wl, step)
        q = wl.draft_q(step)
        bounds = torch.empty((wl.k_pool.shape[0], Hkv, 2, D), dtype=wl.k_pool.dtype, device=DEV)
        s3r.page_bounds_update(kvc, bounds)
        sel, nsel = s3r.page_select(kvc, bounds, q, budget, scale)
        bb = bounds.clone()
        out, sel_b, n_b = s3r.sparse_draft_step(kvc, bb, q, budget, scale,
                                                refresh_from=(wl.seq_lens[step] - 1).contiguous())
        torch.cuda.synchronize()
        L = i32(wl.seq_lens[step])
        rb = oracle.page_bounds(f64(wl.k_pool), i32(wl.page_table), L)
        rsel, rn, rsc = oracle.page_select(rb, f64(q), i32(wl.page_table), L, budget, scale)
        for s_, n_ in ((sel, nsel), (sel_b, n_b)):
            if tied:  # exact: equal scores keep the lowest pages
                assert np.array_equal(i32(s_), rsel) and np.array_equal(i32(n_), rn)
            else:
                check_pages(i32(s_), i32(n_), rsel, rn, rsc, k)
        assert torch.equal(sel, sel_b)
        ref = oracle.sparse_draft_attn(f64(q), f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table), L,
                                       i32(sel_b), scale)
        _check_attn(out, ref, kv)

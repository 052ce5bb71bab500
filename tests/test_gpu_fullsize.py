"""Full-size GPU parity on the benchmark workloads, in the launch configuration
bench.py times (same split plan, same workspaces), checked on sampled
(sequence, kv head) slices the oracle computes one by one.

Per workload: the first draft step (the fused tail-page bounds refresh, page
select and sparse draft attention, as bench.py runs it), the dense verify of
gamma + 1 queries, the speculative sampling of every sequence, the round's
once-per-round selection reused at its last draft step (bench.py's
select_once), and a KV commit of the verify's gamma + 1 rows at the accepted
lengths. Tolerances as in test_gpu_parity.py; the commit is bit-exact.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import self_sparse_speculative_paged_amd as s3r
from s3r_inputs import make_workload
from tests.parity import check_pages, check_tokens

pytestmark = pytest.mark.gpu


def _slice(wl, b, h, G):
    """Host fp64 copies of sequence b's pages for kv head h (data movement only)."""
    n = -(-(int(wl.ctx[b]) + wl.cfg["gamma"]) // wl.cfg["P"])
    idx = wl.page_table[b, :n].long()
    K = wl.k_pool.index_select(0, idx)[:, h:h + 1].to("cpu", torch.float64).numpy()
    V = wl.v_pool.index_select(0, idx)[:, h:h + 1].to("cpu", torch.float64).numpy()
    pt = np.arange(n, dtype=np.int64)[None, :]
    return K, V, pt


def _run_fullsize(name, samples, shrink_to=None):
    torch.manual_seed(0)
    wl = make_workload(name, device="cuda", seed=0)
    cfg = wl.cfg
    if shrink_to is not None:  # keep the longest sequences, as the long tail shrinks
        keep = torch.argsort(wl.ctx, descending=True, stable=True)[:shrink_to].sort().values
        wl.ctx = wl.ctx[keep]
        wl.page_table = wl.page_table[keep.to("cuda")].contiguous()
        wl.seq_lens = [s[keep.to("cuda")].contiguous() for s in wl.seq_lens]
        wl.q_verify = wl.q_verify[keep.to("cuda")].contiguous()
        wl.draft_logits = wl.draft_logits[keep.to("cuda")].contiguous()
        wl.target_logits = wl.target_logits[keep.to("cuda")].contiguous()
        wl.draft_tokens = wl.draft_tokens[keep.to("cuda")].contiguous()
        cfg = dict(cfg, B=shrink_to)
    B, Hq, Hkv, D, P, gamma = (cfg[k] for k in ("B", "Hq", "Hkv", "D", "P", "gamma"))
    G = Hq // Hkv
    budget, k = cfg["budget"], cfg["budget"] // P
    scale = 1.0 / math.sqrt(D)
    total = sum(-(-(int(L) + gamma) // P) for L in wl.ctx)
    kv = s3r.PagedKVCache(wl.k_pool, wl.v_pool, wl.page_table, wl.seq_lens[0], Hq,
                          total_pages_hint=total)
    bounds = torch.empty((wl.k_pool.shape[0], Hkv, 2, D), dtype=wl.k_pool.dtype, device="cuda")
    # bounds as of the full pre-filled KV; the draft step refreshes its tail page
    kv.set_seq_lens(wl.seq_lens[gamma])
    s3r.page_bounds_update(kv, bounds)
    kv.set_seq_lens(wl.seq_lens[0])
    q0 = wl.draft_q(0)
    d_out, sel, nsel = s3r.sparse_draft_step(kv, bounds, q0, budget, scale,
                                             refresh_from=(wl.seq_lens[0] - 1).contiguous())
    kv.set_seq_lens(wl.seq_lens[gamma])
    v_out = s3r.dense_verify_attn(kv, wl.q_verify, scale)
    out, nacc = s3r.spec_sample(wl.draft_logits, wl.target_logits, wl.draft_tokens,
                                cfg["temperature"], 0, 0)
    torch.cuda.synchronize()

    for b, h in samples:
        if b >= B:
            continue
        L = int(wl.ctx[b])
        K, V, pt = _slice(wl, b, h, G)
        heads = slice(h * G, (h + 1) * G)
        # bounds of this slice (exact), as the draft step sees them
        rb = oracle.page_bounds(K, pt, np.array([L]))
        n0 = oracle.n_pages(L, P)
        phys = wl.page_table[b, :n0].long()
        got_b = bounds.index_select(0, phys)[:, h:h + 1].to("cpu", torch.float64).numpy()
        assert np.array_equal(got_b, rb[:n0]), (name, b, h, "bounds")
        # selection
        qd = q0[b:b + 1, heads].to("cpu", torch.float64).numpy()
        rsel, rn, rsc = oracle.page_select(rb, qd, pt, np.array([L]), budget, scale, P)
        gsel = sel[b:b + 1, h:h + 1].cpu().numpy()
        check_pages(gsel, nsel[b:b + 1].cpu().numpy(), rsel, rn, rsc, k)
        # draft attention over the GPU's selection
        rd = oracle.sparse_draft_attn(qd, K, V, pt, np.array([L]), gsel, scale)
        err_d = np.max(np.abs(d_out[b, heads].cpu().numpy() - rd[0]))
        assert err_d <= 1e-2, (name, b, h, "draft", err_d)
        # verify, every query row of the slice
        qv = wl.q_verify[b:b + 1, :, heads].to("cpu", torch.float64).numpy()
        rv = oracle.dense_verify_attn(qv, K, V, pt, np.array([L + gamma]), scale)
        err_v = np.max(np.abs(v_out[b, :, heads].cpu().numpy() - rv[0]))
        assert err_v <= 1e-2, (name, b, h, "verify", err_v)

    # once-per-round selection at step 0, reused at the round's last step
    kv.set_seq_lens(wl.seq_lens[0])
    _, rsel_g, rnsel_g = s3r.sparse_draft_round(kv, bounds, q0, budget, gamma, scale,
                                                refresh_from=(wl.seq_lens[0] - 1).contiguous())
    kv.set_seq_lens(wl.seq_lens[gamma - 1])
    q_last = wl.draft_q(gamma - 1)
    last_out = s3r.sparse_draft_attn(kv, q_last, rsel_g, scale)
    torch.cuda.synchronize()
    for b, h in samples:
        if b >= B:
            continue
        L = int(wl.ctx[b])
        K, V, pt = _slice(wl, b, h, G)
        heads = slice(h * G, (h + 1) * G)
        rb = oracle.page_bounds(K, pt, np.array([L]))
        qd = q0[b:b + 1, heads].to("cpu", torch.float64).numpy()
        rsel, rn, rsc = oracle.page_select_round(rb, qd, pt, np.array([L]), budget, gamma, scale, P)
        g = [int(x) for x in rsel_g[b, h].cpu() if x >= 0]
        r = [int(x) for x in rsel[0, 0] if x >= 0]
        assert int(rnsel_g[b]) == int(rn[0]) and len(g) == len(r), (name, b, h, "round select")
        forced = oracle.round_forced_pages(L, gamma, P, pt.shape[1])
        assert set(forced) <= set(g), (name, b, h, forced)
        if g != r:
            sc = rsc[(0, 0)]
            kth = sorted(sc.values(), reverse=True)[k - len(forced) - 1]
            assert all(abs(sc[j] - kth) <= 1e-4 for j in set(g) ^ set(r)), (name, b, h)
        ql = q_last[b:b + 1, heads].to("cpu", torch.float64).numpy()
        rl = oracle.sparse_draft_attn(ql, K, V, pt, np.array([L + gamma - 1]),
                                      rsel_g[b:b + 1, h:h + 1].cpu().numpy(), scale)
        err_l = np.max(np.abs(last_out[b, heads].cpu().numpy() - rl[0]))
        assert err_l <= 1e-2, (name, b, h, "round draft", err_l)

    # KV commit of gamma + 1 rows from the round's first position, kept up to
    # the accepted length (the rest rolled back)
    first = (wl.seq_lens[0] - 1).contiguous()
    committed = (wl.seq_lens[0] + nacc).contiguous()
    gen = torch.Generator(device="cuda").manual_seed(3)
    k_new = torch.randn((B, gamma + 1, Hkv, D), device="cuda", generator=gen).to(wl.k_pool.dtype)
    v_new = torch.randn((B, gamma + 1, Hkv, D), device="cuda", generator=gen).to(wl.k_pool.dtype)
    before = {}
    for b, h in samples:
        if b < B:
            K, V, pt = _slice(wl, b, h, G)
            n = pt.shape[1]
            phys = wl.page_table[b, :n].long()
            before[(b, h)] = (K, V, pt, bounds.index_select(0, phys)[:, h:h + 1].double().cpu().numpy())
    kv.set_seq_lens(committed)
    s3r.kv_commit(kv, k_new, v_new, first, bounds)
    torch.cuda.synchronize()
    for (b, h), (K, V, pt, B0) in before.items():
        K2, V2, _ = _slice(wl, b, h, G)
        phys = wl.page_table[b, :pt.shape[1]].long()
        B2 = bounds.index_select(0, phys)[:, h:h + 1].double().cpu().numpy()
        rK, rV, rB = oracle.kv_commit(K, V, pt, k_new[b:b + 1, :, h:h + 1].double().cpu().numpy(),
                                      v_new[b:b + 1, :, h:h + 1].double().cpu().numpy(),
                                      first[b:b + 1].cpu().numpy(), committed[b:b + 1].cpu().numpy(),
                                      B0)
        assert np.array_equal(K2, rK) and np.array_equal(V2, rV), (name, b, h, "commit rows")
        assert np.array_equal(B2, rB, equal_nan=True), (name, b, h, "commit bounds")

    ro, rn, dec = oracle.spec_sample(wl.draft_logits.double().cpu().numpy(),
                                     wl.target_logits.double().cpu().numpy(),
                                     wl.draft_tokens.cpu().numpy(), cfg["temperature"], 0, 0)
    full = check_tokens(out.cpu().numpy(), nacc.cpu().numpy(), ro, rn, dec)
    assert full >= B // 2, (full, B)  # vocab-wide draws: a 1e-6 CDF window excludes a few


def test_fullsize_qwen3_8b():
    _run_fullsize("qwen3_8b", [(0, 0), (17, 5), (31, 7)])


def test_fullsize_qwen3_1p7b():
    _run_fullsize("qwen3_1p7b", [(0, 0), (63, 7)])


def test_fullsize_aggressive():
    _run_fullsize("aggressive", [(3, 2), (15, 6)])


@pytest.mark.parametrize("batch", [128, 64, 16, 8])  # the batch sizes bench.py --shrink times
def test_fullsize_ragged(batch):
    _run_fullsize("ragged", [(0, 1), (5, 3), (batch - 1, 7)], shrink_to=batch)

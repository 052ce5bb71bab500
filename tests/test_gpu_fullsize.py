"""Full-size GPU parity on the benchmark workloads, in the launch configuration
bench.py times (same split plan, same workspaces), checked on sampled
(sequence, kv head) slices the oracle computes one by one.

Per workload: the first draft step (the fused tail-page bounds refresh, page
select and sparse draft attention, as bench.py runs it), the dense verify of
gamma + 1 queries, and the speculative sampling of every sequence. Tolerances
as in test_gpu_parity.py.
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
        keep = torch.argsort(wl.ctx, descending=True)[:shrink_to].sort().values
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


@pytest.mark.parametrize("batch", [128, 8])
def test_fullsize_ragged(batch):
    _run_fullsize("ragged", [(0, 1), (5, 3), (batch - 1, 7)], shrink_to=batch)

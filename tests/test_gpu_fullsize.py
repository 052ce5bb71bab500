"""Full-size GPU parity on the benchmark workloads, in the launch configuration
bench.py times (same split plan, same workspaces), checked on every (sequence,
kv head) slice: the oracle runs each slice in a pool of spawned CPU workers
(tests/oracle_pool.py) while the GPU results wait on the host.

Per workload: the first draft step (the fused tail-page bounds refresh, page
select and sparse draft attention, as bench.py runs it), the dense verify of
gamma + 1 queries, the round's once-per-round selection reused at its last
draft step (bench.py's select_once), the drafter's own draws and the
acceptance rate of every draft position, the speculative sampling of every
sequence (with the oracle's stream-2 draws as its draft tokens), and a KV
commit of the verify's gamma + 1 rows at the accepted lengths on sampled
slices (bit-exact). Tolerances as in test_gpu_parity.py and
test_gpu_direct_sampling.py. Where /dev/shm cannot hold the pools, the slice
checks run in this process on a sample that keeps every kv head and the
longest and shortest sequences.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import self_sparse_speculative_paged_amd as s3r
from s3r_inputs import make_workload
from tests import oracle_pool
from tests.parity import check_tokens

pytestmark = pytest.mark.gpu


def _slice(wl, b, h, G):
    """Host fp64 copies of sequence b's pages for kv head h (data movement only)."""
    n = -(-(int(wl.ctx[b]) + wl.cfg["gamma"]) // wl.cfg["P"])
    idx = wl.page_table[b, :n].long()
    K = wl.k_pool.index_select(0, idx)[:, h:h + 1].to("cpu", torch.float64).numpy()
    V = wl.v_pool.index_select(0, idx)[:, h:h + 1].to("cpu", torch.float64).numpy()
    pt = np.arange(n, dtype=np.int64)[None, :]
    return K, V, pt


def _sampled(B, Hkv, ctx, count=16):
    """A seeded sample of slices with every kv head and the longest and shortest sequences."""
    rng = np.random.default_rng(0)
    order = np.argsort(np.asarray(ctx), kind="stable")
    seqs = [int(order[0]), int(order[-1])] + [int(b) for b in rng.integers(0, B, count)]
    return sorted({(b, i % Hkv) for i, b in enumerate(seqs)} | {(int(order[-1]), h) for h in range(Hkv)})


def _run_fullsize(name, shrink_to=None):
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
        cfg = dict(cfg, B=shrink_to)
    B, Hq, Hkv, D, P, gamma = (cfg[k] for k in ("B", "Hq", "Hkv", "D", "P", "gamma"))
    G = Hq // Hkv
    budget, k = cfg["budget"], cfg["budget"] // P
    T = cfg["temperature"]
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
    first = (wl.seq_lens[0] - 1).contiguous()
    d_out, sel, nsel = s3r.sparse_draft_step(kv, bounds, q0, budget, scale, refresh_from=first)
    kv.set_seq_lens(wl.seq_lens[gamma])
    v_out = s3r.dense_verify_attn(kv, wl.q_verify, scale)
    # once-per-round selection at step 0, reused at the round's last step
    kv.set_seq_lens(wl.seq_lens[0])
    _, rsel_g, rnsel_g = s3r.sparse_draft_round(kv, bounds, q0, budget, gamma, scale, refresh_from=first)
    kv.set_seq_lens(wl.seq_lens[gamma - 1])
    q_last = wl.draft_q(gamma - 1)
    last_out = s3r.sparse_draft_attn(kv, q_last, rsel_g, scale)
    torch.cuda.synchronize()
    print(f"{name} B={B}: GPU round done, checking {B * Hkv} slices", flush=True)

    # the drafter's draws (the oracle's stream-2 draws are spec_sample's input), and alpha
    dl = wl.draft_logits.double().cpu().numpy()
    tl = wl.target_logits.double().cpu().numpy()
    x_ref, margin = oracle.draw_tokens(dl, T, 0, 0)
    x_gpu = s3r.draft_sample(wl.draft_logits, T, 0, 0).cpu().numpy()
    close = margin <= 1e-6
    assert np.array_equal(x_gpu[~close], x_ref[~close]), (name, "draft_sample")
    assert (~close).mean() >= 0.5, (name, (~close).mean())
    alpha = s3r.acceptance_rate(wl.draft_logits, wl.target_logits, T).cpu().numpy()
    a_err = np.max(np.abs(alpha - oracle.acceptance_rate(dl, tl, T)))
    assert a_err <= 5e-6, (name, "alpha", a_err)
    x_dev = torch.from_numpy(x_ref).to("cuda")
    out, nacc = s3r.spec_sample(wl.draft_logits, wl.target_logits, x_dev, T, 0, 0)
    torch.cuda.synchronize()

    ctx = [int(L) for L in wl.ctx]
    bounds_bits = bounds.view(torch.int16)
    tasks = []
    for b in range(B):
        L = ctx[b]
        n = -(-(L + gamma) // P)
        phys = wl.page_table[b, :n].long()
        bb = bounds_bits.index_select(0, phys).cpu().numpy().view(np.uint16)
        for h in range(Hkv):
            heads = slice(h * G, (h + 1) * G)
            tasks.append(dict(
                key=(b, h), idx=phys.cpu().numpy(), h=h, L=L, bf16=True, max_pages=wl.page_table.shape[1],
                cfg=dict(P=P, gamma=gamma, budget=budget, D=D),
                bounds=bb[:, h], q0=q0[b, heads].double().cpu().numpy(),
                qv=wl.q_verify[b, :, heads].double().cpu().numpy(),
                sel=sel[b, h].cpu().numpy(), nsel=int(nsel[b]), draft=d_out[b, heads].cpu().numpy(),
                verify=v_out[b, :, heads].cpu().numpy(), round_sel=rsel_g[b, h].cpu().numpy(),
                round_nsel=int(rnsel_g[b]), q_last=q_last[b, heads].double().cpu().numpy(),
                round_draft=last_out[b, heads].cpu().numpy()))
    if oracle_pool.pool_fits(wl.k_pool, wl.v_pool):
        failed, wall = oracle_pool.run(wl.k_pool, wl.v_pool, "check_round_slice", tasks)
        print(f"{name} B={B}: {len(tasks)} slices checked in {wall:.1f} s", flush=True)
    else:
        import warnings
        warnings.warn(f"{name}: /dev/shm cannot hold the pools; checking a sample of slices in-process")
        keep = set(_sampled(B, Hkv, ctx))
        failed = oracle_pool.run_local(wl.k_pool, wl.v_pool, "check_round_slice",
                                       [t for t in tasks if t["key"] in keep])
    assert not failed, (name, B, sorted(failed.items())[:4])

    samples = _sampled(B, Hkv, ctx, count=4)
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

    ro, rn, dec = oracle.spec_sample(dl, tl, x_ref, T, 0, 0)
    full = check_tokens(out.cpu().numpy(), nacc.cpu().numpy(), ro, rn, dec)
    assert full >= B // 2, (full, B)  # vocab-wide draws: a 1e-6 CDF window excludes a few


def test_fullsize_qwen3_8b():
    _run_fullsize("qwen3_8b")


def test_fullsize_qwen3_1p7b():
    _run_fullsize("qwen3_1p7b")


def test_fullsize_aggressive():
    _run_fullsize("aggressive")


@pytest.mark.parametrize("batch", [128, 64, 16, 8])  # the batch sizes bench.py --shrink times
def test_fullsize_ragged(batch):
    _run_fullsize("ragged", shrink_to=batch)

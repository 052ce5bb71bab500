"""The per-slice oracle pool that the full-size GPU tests use, run on the CPU:
a small bf16 round whose results are the oracle's own passes every slice, and
a slice with one planted wrong value is reported (in the pool and in-process)."""
import math

import numpy as np
import torch

import oracle
from s3r_inputs import make_workload
from tests import oracle_pool
from tests.oracle_io import f64, i32


def _tasks():
    cfg = dict(B=3, Hq=4, Hkv=2, D=64, L=None, P=16, budget=64, gamma=3, V=64, kv_dtype="bf16",
               draft_sd=2.0, noise_sd=0.7, temperature=1.0, heavy_pages=0)
    wl = make_workload(cfg, device="cpu", seed=5, ctx=[300, 90, 161], with_logits=False)
    P, gamma, budget, D, G = 16, 3, 64, 64, 2
    scale = 1.0 / math.sqrt(D)
    K, V, pt = f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table)
    L0, Lv, Ll = i32(wl.seq_lens[0]), i32(wl.seq_lens[gamma]), i32(wl.seq_lens[gamma - 1])
    full = oracle.page_bounds(K, pt, Lv)
    b0 = oracle.page_bounds(K, pt, L0)
    bounds = np.where(np.isnan(b0), full, b0)  # the tail page refreshed at L0, the rest pre-filled
    q0 = f64(wl.draft_q(0))
    sel, nsel, _ = oracle.page_select(b0, q0, pt, L0, budget, scale)
    d = oracle.sparse_draft_attn(q0, K, V, pt, L0, sel, scale)
    v = oracle.dense_verify_attn(f64(wl.q_verify), K, V, pt, Lv, scale)
    rsel, rn, _ = oracle.page_select_round(b0, q0, pt, L0, budget, gamma, scale)
    ql = f64(wl.draft_q(gamma - 1))
    last = oracle.sparse_draft_attn(ql, K, V, pt, Ll, rsel, scale)
    bits = torch.from_numpy(bounds.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    tasks = []
    for b in range(3):
        L = int(L0[b])
        n = -(-(L + gamma) // P)
        idx = pt[b, :n]
        for h in range(2):
            hs = slice(h * G, (h + 1) * G)
            tasks.append(dict(key=(b, h), idx=idx, h=h, L=L, bf16=True, max_pages=pt.shape[1],
                              cfg=dict(P=P, gamma=gamma, budget=budget, D=D), bounds=bits[idx, h],
                              q0=q0[b, hs], qv=f64(wl.q_verify)[b, :, hs], sel=sel[b, h], nsel=int(nsel[b]),
                              draft=d[b, hs].astype(np.float32), verify=v[b, :, hs].astype(np.float32),
                              round_sel=rsel[b, h], round_nsel=int(rn[b]), q_last=ql[b, hs],
                              round_draft=last[b, hs].astype(np.float32)))
    return wl, tasks


def test_pool_passes_the_oracles_own_results_and_reports_a_planted_error():
    wl, tasks = _tasks()
    tasks[3]["verify"] = tasks[3]["verify"].copy()
    tasks[3]["verify"][1, 0, 5] += 0.5  # one wrong verify value in slice (1, 1)
    failed, _ = oracle_pool.run(wl.k_pool, wl.v_pool, "check_round_slice", tasks, workers=2)
    assert list(failed) == [(1, 1)] and failed[(1, 1)][0].startswith("verify"), failed
    assert list(oracle_pool.run_local(wl.k_pool, wl.v_pool, "check_round_slice", tasks)) == [(1, 1)]

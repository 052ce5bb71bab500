"""Write tests/golden/tiny_fp32_seed0.json from the oracle alone.

The S3R pages print no worked example, so nothing here is the pages' value:
every stored number is the pinned oracle's output on the seeded tiny fp32
workload (1 layer, B=2, 4 q / 2 kv heads, D=64, context 512, page 16, budget
4 pages, gamma 4, vocab 1024, Philox seed 0). The fixture freezes the oracle so
that a later change to its arithmetic shows up as a failing regression test.
Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from s3r_inputs import make_workload  # noqa: E402
from tests.oracle_io import f64, i32  # noqa: E402


def compute():
    wl = make_workload("tiny_fp32", device="cpu", seed=0)
    c = wl.cfg
    scale = 1.0 / np.sqrt(c["D"])
    K, V, pt = f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table)
    res = {"config": "tiny_fp32", "seed": 0, "steps": []}
    for j in range(c["gamma"]):
        L = i32(wl.seq_lens[j])
        q = f64(wl.draft_q(j))
        bounds = oracle.page_bounds(K, pt, L)
        sel, nsel, _ = oracle.page_select(bounds, q, pt, L, c["budget"], scale)
        o = oracle.sparse_draft_attn(q, K, V, pt, L, sel, scale)
        res["steps"].append({"selected": sel.tolist(), "num_selected": nsel.tolist(),
                             "draft_out_row0": o[:, 0, :8].tolist()})
    L = i32(wl.seq_lens[c["gamma"]])
    ov = oracle.dense_verify_attn(f64(wl.q_verify), K, V, pt, L, scale)
    res["verify_out_head0"] = ov[:, :, 0, :8].tolist()
    out, n, _ = oracle.spec_sample(f64(wl.draft_logits), f64(wl.target_logits),
                                   i32(wl.draft_tokens), c["temperature"], 0, 0)
    res["out_tokens"] = out.tolist()
    res["num_accepted"] = n.tolist()
    return res


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_seed0.json")
    with open(path, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", path)

"""bench.py's algorithmic byte count: the numerator of `value` and of the
roofline's `achieved`.

The count is recomputed here from its per-unit definition, not from bench.py's
loop. One bf16 token of K+V is 2*Hkv*D*2 bytes, and one page's min/max bounds
take the same. A sequence reads:
- at each draft step, its bounds (one per page present) and the selected
  pages' K+V;
- at verify, every token's K+V;
- in the sampler, 2*gamma + 1 fp32 logit rows.
The totals are also pinned to the workloads' GB figures, to three significant
digits.
"""
import math

import pytest

import bench
from s3r_inputs import CONFIGS


def _closed_form(cfg, L, B, select_once):
    P, D, Hkv, gamma, V = (cfg[k] for k in ("P", "D", "Hkv", "gamma", "V"))
    tok = 2 * Hkv * D * 2
    k = cfg["budget"] // P
    pages = [math.ceil((L + j) / P) for j in range(gamma)]
    select = (pages[0] if select_once else sum(pages)) * tok * B
    draft = sum(min(k, n) for n in pages) * P * tok * B
    verify = (L + gamma) * tok * B
    sample = (2 * gamma + 1) * V * 4 * B
    return dict(select=select, draft=draft, verify=verify, sample=sample)


@pytest.mark.parametrize("name,verify_gb,select_gb,draft_gb,sample_gb,chain_gb,once_gb", [
    ("qwen3_1p7b", 2.148, 0.537, 1.074, 0.350, 4.109, 3.707),
    ("qwen3_8b", 4.296, 1.611, 1.611, 0.253, 7.770, 6.428),
    ("aggressive", 4.296, 2.147, 0.134, 0.165, 6.743, 4.864),
])
def test_round_bytes_match_the_per_unit_model(name, verify_gb, select_gb, draft_gb, sample_gb, chain_gb,
                                              once_gb):
    cfg = CONFIGS[name]
    B, L = cfg["B"], cfg["L"]
    ctx = [L] * B
    got = bench.step_bytes(cfg, ctx)
    once = bench.step_bytes(cfg, ctx, select_once=True)
    for key, want in _closed_form(cfg, L, B, False).items():
        assert got[key] == want, (name, key)
    for key, want in _closed_form(cfg, L, B, True).items():
        assert once[key] == want, (name, key)
    for key, gb in (("verify", verify_gb), ("select", select_gb), ("draft", draft_gb), ("sample", sample_gb)):
        assert abs(got[key] / 1e9 - gb) <= 0.0015, (name, key, got[key])
    chain = sum(got[k] for k in ("select", "draft", "verify", "sample"))
    chain_once = sum(once[k] for k in ("select", "draft", "verify", "sample"))
    assert abs(chain / 1e9 - chain_gb) <= 0.0015 and abs(chain_once / 1e9 - once_gb) <= 0.0015
    # tail-page refreshes and q/o: well under 1% of the round
    small = got["bounds"] + got["q_out"]
    assert 0 < small < 0.01 * sum(got.values())


def test_ragged_bytes_follow_each_sequence():
    cfg = CONFIGS["ragged"]
    ctx = [2048, 8192, 65536, 3001]
    got = bench.step_bytes(cfg, ctx)
    want = {key: 0 for key in ("select", "draft", "verify", "sample")}
    for L in ctx:
        for key, v in _closed_form(cfg, L, 1, False).items():
            want[key] += v
    for key, v in want.items():
        assert got[key] == v, key


def test_verify_flops_and_the_mfma_counter():
    """The verify's algorithmic flops at the 8B shape (4 flops per query row,
    visible position and d), and the bf16 MFMA flops rocprofv3 counted per
    verify launch (profiles/) against what the kernel issues by design: rows
    padded to 16-row blocks (28 -> 32), two MFMAs per P.V block (P split into a
    hi and a lo bf16 part) and whole 32-token windows (2049 pages -> 1025)."""
    import os

    cfg = CONFIGS["qwen3_8b"]
    B, L, gamma, D, Hq, Hkv = (cfg[k] for k in ("B", "L", "gamma", "D", "Hq", "Hkv"))
    assert bench.verify_algorithmic_flops(cfg, [L] * B) == 4 * D * Hq * B * (7 * 32768 + 21) == 120270094336
    path = os.path.join(os.path.dirname(bench.__file__), "profiles", "counters_mfma_dense_verify_qwen3_8b.txt")
    fields = dict(line.split(":", 1) for line in open(path) if ":" in line)
    counted = int(fields["mfma_flops_bf16_per_launch"])
    rows = 32                                   # 28 rows in two 16-row blocks
    windows = math.ceil(math.ceil((L + gamma) / cfg["P"]) / 2)
    per_row_token = 2 * D + 2 * (2 * D)         # S = K.Q^T, then P_hi.V and P_lo.V
    assert counted == per_row_token * rows * 32 * windows * B * Hkv
    assert 0 < float(fields["mfma_util_pct"]) < 100

"""bench.py's cpu_baseline leg on a small workload, on the CPU: the pooled run
over shared memory and the one-process run it falls back to when /dev/shm is
too small both cover the whole round, and the bytes they count are the
round's algorithmic bytes (bounds, draft pages, verify, sampler logits)."""
import pytest

import bench
from s3r_inputs import make_workload

CFG = dict(B=3, Hq=4, Hkv=2, D=64, L=None, P=16, budget=64, gamma=3, V=100, kv_dtype="bf16",
           draft_sd=2.0, noise_sd=0.7, temperature=1.0, heavy_pages=0)
CTX = [300, 77, 129]


@pytest.mark.parametrize("pooled", [True, False], ids=["pooled", "one_process"])
def test_cpu_baseline_counts_the_whole_round(pooled, monkeypatch):
    if not pooled:
        monkeypatch.setattr(bench, "_shm_free_bytes", lambda: 0)
    wl = make_workload(CFG, device="cpu", seed=4, ctx=CTX)
    got = bench.cpu_baseline(wl, CFG, budget_s=120.0)
    want = bench.step_bytes(CFG, CTX)
    assert got["bytes"] == sum(want[k] for k in ("select", "draft", "verify", "sample"))
    assert got["kind"] == "oracle" and got["value"] > 0 and got["unit"] == "GB/s"
    assert got["sample"].startswith(f"{CFG['B'] * CFG['Hkv']} of the {CFG['B'] * CFG['Hkv']}")
    assert (got["cores"] == 1) == (not pooled)

"""The seeded input recipe (s3r_inputs), checked on the CPU.

The workloads stand in for the pages' RL rollouts, so their shapes and laws are
part of what the benchmark and the parity tests claim:
- every configuration has the shapes of its description;
- ragged lengths follow the clipped lognormal recipe;
- each sequence owns its own physical pages, and together they tile the pool;
- heavy pages are whole pages with keys scaled by 4, the same for every kv head;
- K/V/Q are N(0, 1) rounded to the KV dtype;
- the logits follow draft ~ N(0, sd_d) and target = draft + N(0, sd_n), and the
  bonus row has the same marginal;
- draft tokens are draws from softmax(draft / T);
- a seed reproduces its tensors.
"""
import math

import numpy as np
import pytest
import torch

from s3r_inputs import CONFIGS, make_workload, ragged_lengths


def _small(**kw):
    cfg = dict(CONFIGS["tiny_fp32"])
    cfg.update(kw)
    return cfg


@pytest.mark.parametrize("name,shape", [
    ("tiny_fp32", dict(B=2, Hq=4, Hkv=2, D=64, L=512, P=16, budget=64, gamma=4, V=1024, kv_dtype="f32",
                       draft_sd=1.5, noise_sd=0.5, temperature=1.0, heavy_pages=0)),
    ("qwen3_1p7b", dict(B=64, Hq=16, Hkv=8, D=128, L=8192, P=16, budget=1024, gamma=4, V=151936,
                        kv_dtype="bf16", draft_sd=2.0, noise_sd=0.7)),
    ("qwen3_8b", dict(B=32, Hq=32, Hkv=8, D=128, L=32768, P=16, budget=2048, gamma=6, V=151936,
                      kv_dtype="bf16", draft_sd=2.0, noise_sd=0.5, heavy_pages=4)),
    ("ragged", dict(B=128, Hq=32, Hkv=8, D=128, L=None, P=16, budget=2048, gamma=4, kv_dtype="bf16",
                    shrink=(128, 64, 16, 8))),
    ("aggressive", dict(B=16, Hq=32, Hkv=8, D=128, L=65536, P=16, budget=256, gamma=8, kv_dtype="bf16",
                        noise_sd=1.35)),
])
def test_configs_have_their_described_shapes(name, shape):
    cfg = CONFIGS[name]
    for key, want in shape.items():
        assert cfg[key] == want, (name, key, cfg[key], want)


def test_ragged_lengths_follow_the_clipped_lognormal():
    n = 20000
    ctx = ragged_lengths(n, seed=3).numpy().astype(np.int64)
    assert ctx.min() >= 2048 and ctx.max() <= 65536
    assert abs(np.median(ctx) / 8192 - 1) < 0.03
    # clip masses: P(z < ln(1/4)/0.8) and P(z > ln(8)/0.8) for z ~ N(0, 1)
    lo = 0.5 * math.erfc(math.log(4) / 0.8 / math.sqrt(2))
    hi = 0.5 * math.erfc(math.log(8) / 0.8 / math.sqrt(2))
    for got, want in ((np.mean(ctx == 2048), lo), (np.mean(ctx == 65536), hi)):
        assert abs(got - want) <= 4 * math.sqrt(want * (1 - want) / n) + 1e-4, (got, want)
    assert np.array_equal(ragged_lengths(128, seed=0).numpy(), ragged_lengths(128, seed=0).numpy())


def test_page_tables_tile_the_pool():
    ctx = [300, 17, 1, 95, 512]
    wl = make_workload(_small(B=5), seed=2, ctx=ctx, with_logits=False)
    P, gamma = wl.cfg["P"], wl.cfg["gamma"]
    pt = wl.page_table.numpy()
    used = []
    for b, L in enumerate(ctx):
        n = -(-(L + gamma) // P)
        row = pt[b, :n].tolist()
        assert len(set(row)) == n
        used += row
    assert sorted(used) == list(range(wl.k_pool.shape[0]))  # disjoint, and every page used
    assert wl.k_pool.shape[0] == sum(-(-(L + gamma) // P) for L in ctx)
    assert [int(s[0]) for s in wl.seq_lens] == [300 + j for j in range(gamma + 1)]


def test_heavy_pages_are_whole_pages_with_keys_times_four():
    cfg = _small(B=3, kv_dtype="bf16", heavy_pages=4)
    ctx = [300, 200, 77]
    heavy = make_workload(cfg, seed=5, ctx=ctx, with_logits=False)
    plain = make_workload(dict(cfg, heavy_pages=0), seed=5, ctx=ctx, with_logits=False)
    assert torch.equal(heavy.page_table, plain.page_table) and torch.equal(heavy.v_pool, plain.v_pool)
    scaled = set()
    for b, L in enumerate(ctx):
        pages = heavy.heavy[b].tolist()
        assert len(set(pages)) == 4
        assert all(0 <= j < (L + cfg["gamma"]) // cfg["P"] for j in pages)  # complete pages only
        scaled |= {int(heavy.page_table[b, j]) for j in pages}
    for p in range(heavy.k_pool.shape[0]):  # every kv head of a heavy page, and nothing else
        want = (plain.k_pool[p].float() * 4).to(torch.bfloat16) if p in scaled else plain.k_pool[p]
        assert torch.equal(heavy.k_pool[p], want), p


def test_kv_and_queries_are_rounded_standard_normals():
    wl = make_workload(_small(B=4, kv_dtype="bf16", L=2000), seed=1, with_logits=False)
    for t in (wl.k_pool, wl.v_pool, wl.q_verify):
        assert t.dtype == torch.bfloat16
        x = t.float().flatten()
        assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1) < 0.02


def test_logits_follow_the_recipe():
    cfg = _small(B=8, V=8192, gamma=4, draft_sd=2.0, noise_sd=0.7)
    wl = make_workload(cfg, seed=4, ctx=[64] * 8)
    d, t = wl.draft_logits.double(), wl.target_logits.double()
    g = cfg["gamma"]
    assert d.shape == (8, g, 8192) and t.shape == (8, g + 1, 8192)
    assert abs(float(d.std()) / 2.0 - 1) < 0.02
    assert abs(float((t[:, :g] - d).std()) / 0.7 - 1) < 0.02
    assert abs(float(t[:, g].std()) / math.hypot(2.0, 0.7) - 1) < 0.03  # the bonus row's marginal


def test_draft_tokens_are_draws_from_the_draft_distribution():
    cfg = _small(B=4000, V=5, gamma=1, draft_sd=1.0, temperature=0.8)
    wl = make_workload(cfg, seed=6, ctx=[16] * 4000)
    p = torch.softmax(wl.draft_logits.double() / 0.8, dim=-1)[:, 0]       # [B][V]
    x = wl.draft_tokens[:, 0].long()
    assert int(x.min()) >= 0 and int(x.max()) < 5
    freq = torch.bincount(x, minlength=5).double() / 4000
    want = p.mean(dim=0)
    sd = torch.sqrt((p * (1 - p)).sum(dim=0)) / 4000
    assert torch.all((freq - want).abs() <= 5 * sd), (freq, want)


def test_a_seed_reproduces_its_workload():
    a = make_workload("tiny_fp32", seed=9)
    b = make_workload("tiny_fp32", seed=9)
    c = make_workload("tiny_fp32", seed=10)
    for name in ("k_pool", "v_pool", "page_table", "q_verify", "draft_logits", "target_logits", "draft_tokens"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert not torch.equal(a.k_pool, c.k_pool)

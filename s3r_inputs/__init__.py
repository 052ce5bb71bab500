"""Seeded synthetic workloads for the S3R hot path.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no attention, no page scoring, no sampling rule). The same
tensors feed the CPU oracle and the HIP library. Random numbers the method
itself consumes (the sampler's uniforms) are not drawn here: both sides derive
them from Philox4x64-10 coordinates.

Layouts (shared with the library's header):
  k_pool [N_phys][Hkv][P][D]     v_pool [N_phys][Hkv][D][P] (value transposed per page)
  page_table [B][max_pages] int32 (physical page ids, randomly permuted over one pool)
  q_verify [B][gamma+1][Hq][D]; the draft query of step j is q_verify[:, j]
  draft_logits [B][gamma][V] fp32, target_logits [B][gamma+1][V] fp32
  draft_tokens [B][gamma] int32, drawn from softmax(draft/T) by Gumbel-max
Positions: a round starts at committed length L_b; the KV is pre-filled for
positions < L_b + gamma. Draft step j sees seq_len = L_b + j, verify sees
seq_len = L_b + gamma with gamma + 1 queries.
"""
from __future__ import annotations

import dataclasses
import math

import torch

__all__ = ["CONFIGS", "Workload", "make_workload", "ragged_lengths"]

# Workload shapes. N(mu, x) in the recipes means standard deviation x.
CONFIGS = {
    # 1 layer, fp32 KV: the small case the oracle runs in seconds.
    "tiny_fp32": dict(B=2, Hq=4, Hkv=2, D=64, L=512, P=16, budget=64, gamma=4,
                      V=1024, kv_dtype="f32", draft_sd=1.5, noise_sd=0.5,
                      temperature=1.0, heavy_pages=0),
    # Qwen3-1.7B-shaped attention layer.
    "qwen3_1p7b": dict(B=64, Hq=16, Hkv=8, D=128, L=8192, P=16, budget=1024, gamma=4,
                       V=151936, kv_dtype="bf16", draft_sd=2.0, noise_sd=0.7,
                       temperature=1.0, heavy_pages=0),
    # Qwen3-8B-shaped attention layer with 4 planted high-norm pages per sequence.
    "qwen3_8b": dict(B=32, Hq=32, Hkv=8, D=128, L=32768, P=16, budget=2048, gamma=6,
                     V=151936, kv_dtype="bf16", draft_sd=2.0, noise_sd=0.5,
                     temperature=1.0, heavy_pages=4),
    # RL long tail: lognormal lengths 2k..64k (median 8k), shared permuted pool.
    "ragged": dict(B=128, Hq=32, Hkv=8, D=128, L=None, P=16, budget=2048, gamma=4,
                   V=151936, kv_dtype="bf16", draft_sd=2.0, noise_sd=0.5,
                   temperature=1.0, heavy_pages=0, shrink=(128, 64, 16, 8)),
    # Aggressive sparse budget; logit noise set for ~0.5 per-token acceptance.
    "aggressive": dict(B=16, Hq=32, Hkv=8, D=128, L=65536, P=16, budget=256, gamma=8,
                       V=151936, kv_dtype="bf16", draft_sd=2.0, noise_sd=1.35,
                       temperature=1.0, heavy_pages=0),
}

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Workload:
    cfg: dict
    ctx: torch.Tensor            # [B] int32 committed length L_b (host)
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    page_table: torch.Tensor     # [B][max_pages] int32
    seq_lens: list               # seq_lens[j] = L + j, j = 0..gamma, int32 [B] each
    q_verify: torch.Tensor       # [B][gamma+1][Hq][D]
    draft_logits: torch.Tensor   # [B][gamma][V] fp32
    target_logits: torch.Tensor  # [B][gamma+1][V] fp32
    draft_tokens: torch.Tensor   # [B][gamma] int32
    heavy: torch.Tensor | None   # [B][n_heavy] logical page ids with scaled keys

    @property
    def max_pages(self):
        return self.page_table.shape[1]

    def draft_q(self, j):
        return self.q_verify[:, j].contiguous()


def ragged_lengths(n, seed=0, median=8192, sigma=0.8, lo=2048, hi=65536):
    """Context lengths clip(round(exp(N(ln median, sigma))), lo, hi), seeded."""
    g = torch.Generator().manual_seed(seed)
    z = torch.randn(n, generator=g, dtype=torch.float64)
    ctx = torch.exp(math.log(median) + sigma * z).round().clamp(lo, hi)
    return ctx.to(torch.int32)


def _randn(shape, gen, device, dtype, chunk=1 << 26):
    """N(0,1) drawn in fp32 then rounded to `dtype` (round-to-nearest-even)."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk):
        e = min(s + chunk, flat.numel())
        flat[s:e] = torch.randn(e - s, generator=gen, device=device).to(dtype)
    return out


def make_workload(cfg, device="cpu", seed=0, ctx=None, with_logits=True, **overrides):
    """Build one seeded workload. `cfg` is a name in CONFIGS or a dict.

    ctx: optional per-sequence committed lengths (list or tensor) overriding L.
    Tensors are created on `device` with a generator seeded from `seed`; the same
    seed on the same device type reproduces the same tensors.
    """
    cfg = dict(CONFIGS[cfg]) if isinstance(cfg, str) else dict(cfg)
    cfg.update(overrides)
    B, Hq, Hkv, D, P, gamma = (cfg[k] for k in ("B", "Hq", "Hkv", "D", "P", "gamma"))
    dt = _DTYPES[cfg["kv_dtype"]]
    dev = torch.device(device)
    gen = torch.Generator(device=dev).manual_seed(seed)
    ghost = torch.Generator().manual_seed(seed + 7919)  # host-side integer draws

    if ctx is None:
        if cfg.get("L") is None:
            ctx = ragged_lengths(B, seed=seed)
        else:
            ctx = torch.full((B,), cfg["L"], dtype=torch.int32)
    ctx = torch.as_tensor(ctx, dtype=torch.int32).cpu()
    assert ctx.numel() == B
    total = ctx + gamma
    npages = [(-(-int(t) // P)) for t in total]
    max_pages = max(npages)
    n_phys = sum(npages)

    # One shared pool; every sequence's pages are a random subset of it.
    perm = torch.randperm(n_phys, generator=ghost).to(torch.int32)
    page_table = torch.zeros((B, max_pages), dtype=torch.int32)
    off = 0
    for b in range(B):
        page_table[b, :npages[b]] = perm[off:off + npages[b]]
        off += npages[b]

    k_pool = _randn((n_phys, Hkv, P, D), gen, dev, dt)
    v_pool = _randn((n_phys, Hkv, D, P), gen, dev, dt)

    heavy = None
    nh = cfg.get("heavy_pages", 0)
    if nh:
        heavy = torch.zeros((B, nh), dtype=torch.int64)
        for b in range(B):
            full = int(total[b]) // P          # complete pages only, never the tail
            heavy[b] = torch.randperm(full, generator=ghost)[:nh]
            phys = page_table[b, heavy[b]].long().to(dev)
            k_pool[phys] = (k_pool[phys].float() * 4.0).to(dt)

    q_verify = _randn((B, gamma + 1, Hq, D), gen, dev, dt)
    seq_lens = [(ctx + j).to(torch.int32).to(dev) for j in range(gamma + 1)]

    draft_logits = target_logits = draft_tokens = None
    if with_logits:
        V = cfg["V"]
        T = cfg["temperature"]
        draft_logits = torch.randn((B, gamma, V), generator=gen, device=dev) * cfg["draft_sd"]
        target_logits = torch.empty((B, gamma + 1, V), device=dev)
        target_logits[:, :gamma] = draft_logits + torch.randn(
            (B, gamma, V), generator=gen, device=dev) * cfg["noise_sd"]
        # the bonus row has no draft partner: same marginal law as the others
        target_logits[:, gamma] = (torch.randn((B, V), generator=gen, device=dev) * cfg["draft_sd"]
                                   + torch.randn((B, V), generator=gen, device=dev) * cfg["noise_sd"])
        # The drafter's own samples x_i ~ softmax(draft_i / T), by Gumbel-max.
        u = torch.rand((B, gamma, V), generator=gen, device=dev, dtype=torch.float64)
        u = u.clamp_min(1e-300)
        gumbel = -torch.log(-torch.log(u))
        draft_tokens = torch.argmax(draft_logits.double() / T + gumbel, dim=-1).to(torch.int32)

    return Workload(cfg=cfg, ctx=ctx, k_pool=k_pool, v_pool=v_pool,
                    page_table=page_table.to(dev), seq_lens=seq_lens, q_verify=q_verify,
                    draft_logits=draft_logits, target_logits=target_logits,
                    draft_tokens=draft_tokens, heavy=heavy)

"""Rounds captured in a HIP graph replay to exactly the eager results.

bench.py times whole rounds as graph replays, so a round is captured once
here (gamma draft steps, verify and sampling; and the select-once variant)
and replayed three times. Between replays the program does its own eager
work: other library calls on other buffers, and synchronisations. Every
output of every replay must equal the eager run bit for bit. The draft steps
refresh the tail-page bounds in place, and that refresh is idempotent.
The ragged batch also puts the longest-first ordering kernel into the graph.
A KV commit, idempotent for the same rows, is replayed the same way.
"""
import numpy as np
import pytest
import torch

import self_sparse_speculative_paged_amd as s3r
from s3r_inputs import make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _workload(ragged):
    rng = np.random.default_rng(5)
    if ragged:  # a few long sequences among many short ones
        ctx = [int(x) for x in rng.choice([120, 260, 500], size=32)]
        ctx[3], ctx[17] = 6000, 4200
    else:
        ctx = [int(x) for x in rng.integers(300, 3000, size=32)]
    cfg = dict(B=32, Hq=32, Hkv=8, D=128, L=None, P=16, budget=512, gamma=4, V=8192,
               kv_dtype="bf16", draft_sd=2.0, noise_sd=0.7, temperature=1.0, heavy_pages=2)
    return make_workload(cfg, device=DEV, seed=9, ctx=ctx)


class Round:
    def __init__(self, wl):
        c = wl.cfg
        self.wl, self.g = wl, c["gamma"]
        B, Hq, Hkv, D, P = c["B"], c["Hq"], c["Hkv"], c["D"], c["P"]
        self.budget, self.k = c["budget"], c["budget"] // P
        self.scale = 1.0 / np.sqrt(D)
        total = sum(-(-(int(L) + self.g) // P) for L in wl.ctx)
        self.kv = s3r.PagedKVCache(wl.k_pool, wl.v_pool, wl.page_table, wl.seq_lens[0], Hq,
                                   total_pages_hint=total)
        self.bounds = torch.zeros((wl.k_pool.shape[0], Hkv, 2, D), dtype=wl.k_pool.dtype, device=DEV)
        s3r.page_bounds_update(self.kv, self.bounds)
        self.first = [(s - 1).contiguous() for s in wl.seq_lens]
        self.q = [wl.draft_q(j) for j in range(self.g)]
        e = lambda *shape, dt=torch.float32: torch.empty(shape, dtype=dt, device=DEV)
        self.sel, self.nsel = e(B, Hkv, self.k, dt=torch.int32), e(B, dt=torch.int32)
        self.d_out = e(self.g, B, Hq, D, dt=torch.bfloat16)
        self.v_out = e(B, self.g + 1, Hq, D, dt=torch.bfloat16)
        self.tok, self.nacc = e(B, self.g + 1, dt=torch.int32), e(B, dt=torch.int32)
        u8 = lambda n: torch.empty(max(1, n), dtype=torch.uint8, device=DEV)
        self.ws_step = u8(s3r.sparse_draft_step_workspace(self.kv, self.budget))
        self.ws_d = u8(s3r.attn_workspace(self.kv, 1, self.k))
        self.ws_v = u8(s3r.attn_workspace(self.kv, self.g + 1, wl.max_pages))
        self.ws_s = u8(s3r.spec_sample_workspace(B, self.g, c["V"]))

    def outputs(self):
        return [self.sel, self.nsel, self.d_out, self.v_out, self.tok, self.nacc, self.bounds]

    def verify_and_sample(self):
        self.kv.set_seq_lens(self.wl.seq_lens[self.g])
        s3r.dense_verify_attn(self.kv, self.wl.q_verify, self.scale, out=self.v_out, workspace=self.ws_v)
        s3r.spec_sample(self.wl.draft_logits, self.wl.target_logits, self.wl.draft_tokens, 1.0, 4, 1,
                        out_tokens=self.tok, num_accepted=self.nacc, workspace=self.ws_s)

    def step(self, j):
        self.kv.set_seq_lens(self.wl.seq_lens[j])
        s3r.sparse_draft_step(self.kv, self.bounds, self.q[j], self.budget, self.scale,
                              refresh_from=self.first[j], selected=self.sel, num_selected=self.nsel,
                              out=self.d_out[j], workspace=self.ws_step)

    def per_step(self):
        for j in range(self.g):
            self.step(j)
        self.verify_and_sample()

    def select_once(self):
        self.kv.set_seq_lens(self.wl.seq_lens[0])
        s3r.sparse_draft_round(self.kv, self.bounds, self.q[0], self.budget, self.g, self.scale,
                               refresh_from=self.first[0], selected=self.sel, num_selected=self.nsel,
                               out=self.d_out[0], workspace=self.ws_step)
        for j in range(1, self.g):
            self.kv.set_seq_lens(self.wl.seq_lens[j])
            s3r.sparse_draft_attn(self.kv, self.q[j], self.sel, self.scale, out=self.d_out[j],
                                  workspace=self.ws_d)
        self.verify_and_sample()


def _same(a, b):
    """Bitwise equality (NaN payloads included)."""
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the capture stream, as bench.py does
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        fn()
    return g


def _eager_noise(r):
    """The program's own work between replays: a library call into other buffers."""
    kv = s3r.PagedKVCache(r.wl.k_pool, r.wl.v_pool, r.wl.page_table, r.wl.seq_lens[1], r.wl.cfg["Hq"])
    s3r.dense_verify_attn(kv, r.wl.q_verify, 0.05)
    torch.cuda.synchronize()


@pytest.mark.parametrize("ragged", [False, True], ids=["uniform", "ragged"])
@pytest.mark.parametrize("variant", ["per_step", "select_once"])
def test_round_graph_replays_equal_eager(ragged, variant):
    print(f"graph replay: {variant}, ragged={ragged}, B=32 Hkv=8 G=4 D=128", flush=True)
    r = Round(_workload(ragged))
    run = getattr(r, variant)
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in r.outputs()]
    g = _capture(run)
    for rep in range(3):
        for t in r.outputs()[:-1]:  # outputs (not the bounds) start from garbage
            t.fill_(-3 if t.dtype == torch.int32 else 7.0)
        _eager_noise(r)
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(r.outputs(), ref)):
            assert _same(a, b), (variant, ragged, rep, i)


def test_kv_commit_graph_replays_equal_eager():
    print("graph replay: kv_commit, B=32 Hkv=8 D=128", flush=True)
    r = Round(_workload(False))
    gen = torch.Generator(device=DEV).manual_seed(2)
    k_new = torch.randn((32, 5, 8, 128), device=DEV, generator=gen).to(torch.bfloat16)
    v_new = torch.randn((32, 5, 8, 128), device=DEV, generator=gen).to(torch.bfloat16)
    committed = (r.wl.seq_lens[0] + 2).contiguous()
    kv = s3r.PagedKVCache(r.wl.k_pool, r.wl.v_pool, r.wl.page_table, committed, 32)

    def commit():
        s3r.kv_commit(kv, k_new, v_new, r.first[0], r.bounds)

    commit()
    torch.cuda.synchronize()
    ref = [r.wl.k_pool.clone(), r.wl.v_pool.clone(), r.bounds.clone()]
    g = _capture(commit)
    for rep in range(3):
        _eager_noise(r)
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip([r.wl.k_pool, r.wl.v_pool, r.bounds], ref)):
            assert _same(a, b), (rep, i)

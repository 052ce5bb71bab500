"""Benchmark one S3R round (the whole hot path) on one MI355X.

A step is one round of "S3R: Fast and Faithful RL Rollouts via
Self-Sparse Speculative Decoding" (Abstract) for one attention layer:
  for j in 0..gamma-1: sparse_draft_step = tail-page bounds refresh ->
                       page select -> sparse draft attention (query L-1+j)
  dense_verify_attn (gamma+1 causal queries over the complete KV)
  spec_sample (accept/reject, residual or bonus draw)
over the Qwen3-8B-shaped layer: bf16 paged KV, 32 q / 8 kv heads, head dim 128,
batch 32, context 32768, page 16, budget 2048 tokens, gamma 6, vocab 151936,
4 planted high-norm pages per sequence. Inputs are seeded synthetic tensors,
resident in HBM before timing. The step is captured once into a HIP graph
and replayed.

Prints one JSON line. `value` is the step's algorithmic HBM bytes (KV, page
bounds and logits each counted once) over the measured step time, in GB/s;
`accepted_tokens_per_s` is committed tokens (accepted + 1 per sequence) per
second. `roofline` covers the dominant launch (dense verify), timed with HIP
events on the stream it runs on; `cpu_baseline` is the fp64 oracle on a
bounded slice of the same workload, on the host. `select_once` times the same
round with one selection per round (s3r_sparse_draft_round at step 0, the
later steps reusing it).

--sweep instead measures the speedup condition over gamma x budget x
acceptance x context at the 8B head shape: per point, the round (both
selection frequencies), a dense single-query decode over the same KV (the
one-layer autoregressive step), the committed tokens per round E, and the
speedup E * t_dense / t_round next to the byte model's E * bytes_dense /
bytes_round. One JSON line per point.

--shrink runs the ragged long-tail batch as it drains: the round on its
longest 128, 64, 16 and 8 sequences, one JSON line per active batch size.

--fidelity compares direct sparse sampling with S3R per budget: a fixed random
head maps the dense and the sparse attention outputs to logits p and q; direct
sparse sampling (s3r_draft_sample) is TV(p, q) = 1 - alpha away from the dense
policy per token, with alpha = sum min(p, q) from s3r_acceptance_rate, while S3R
keeps p's law and accepts at alpha, which s3r_spec_sample measures.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "draft+verify attention KV GB/s (% of HBM peak); accepted tokens/s at 1 GPU"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default="qwen3_8b")
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="time the headline workload only (not the other workloads of the bench line)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="wall-time budget of the oracle baseline's worker-pool phase")
    p.add_argument("--sweep", action="store_true",
                   help="speedup-condition sweep instead of the one-round measurement")
    p.add_argument("--shrink", action="store_true",
                   help="the ragged batch as it drains: rounds on its longest 128, 64, 16 and 8 sequences")
    p.add_argument("--fidelity", action="store_true",
                   help="direct sparse sampling (TV) against S3R's measured acceptance, per budget")
    return p.parse_args()


def verify_algorithmic_flops(cfg, ctx):
    """Flops of one dense verify by definition: query i of a sequence at
    committed length L sees L + i positions, and each (q head, position) costs
    2*D for q.k and 2*D for p*v."""
    D, Hq, gamma = cfg["D"], cfg["Hq"], cfg["gamma"]
    return sum(4 * D * Hq * sum(L + i for i in range(gamma + 1)) for L in ctx)


def step_bytes(cfg, ctx, select_once=False):
    """Algorithmic HBM bytes of one round, summed over sequences. With
    select_once the bounds are read (and the tail page refreshed) at draft
    step 0 only; the later steps reuse that selection."""
    P, D, Hkv, Hq, gamma, V = (cfg[k] for k in ("P", "D", "Hkv", "Hq", "gamma", "V"))
    esz = 2 if cfg["kv_dtype"] == "bf16" else 4
    kv_tok = 2 * Hkv * D * esz                  # K + V of one token, all kv heads
    bound_page = 2 * Hkv * D * esz              # min + max of one page, all kv heads
    k = cfg["budget"] // P
    parts = dict(select=0, draft=0, bounds=0, verify=0, sample=0, q_out=0)
    for L in ctx:
        for j in range(gamma):
            n = -(-(L + j) // P)
            if j == 0 or not select_once:
                parts["select"] += n * bound_page
                parts["bounds"] += P * Hkv * D * esz + bound_page   # tail page read + write
            parts["draft"] += min(k, n) * P * kv_tok
            parts["q_out"] += 2 * Hq * D * esz
        parts["verify"] += (L + gamma) * kv_tok
        parts["q_out"] += 2 * (gamma + 1) * Hq * D * esz
        parts["sample"] += (2 * gamma + 1) * V * 4
    return parts


def build_round(config, dev, seed=0, **overrides):
    """Buffers and launch closures of one round on a fresh seeded workload."""
    import types

    import torch

    import self_sparse_speculative_paged_amd as s3r
    from s3r_inputs import make_workload

    wl = make_workload(config, device=dev, seed=seed, **overrides)
    cfg = wl.cfg
    B, Hq, Hkv, D, P, gamma, V = (cfg[k] for k in ("B", "Hq", "Hkv", "D", "P", "gamma", "V"))
    budget, T = cfg["budget"], cfg["temperature"]
    k = budget // P
    scale = 1.0 / math.sqrt(D)
    ctx = [int(x) for x in wl.ctx]
    total_pages = sum(-(-(L + gamma) // P) for L in ctx)

    kv = s3r.PagedKVCache(wl.k_pool, wl.v_pool, wl.page_table, wl.seq_lens[0], Hq,
                          total_pages_hint=total_pages)
    n_phys = wl.k_pool.shape[0]
    bounds = torch.empty((n_phys, Hkv, 2, D), dtype=wl.k_pool.dtype, device=dev)
    s3r.page_bounds_update(kv, bounds)  # set-up: every page
    first_pos = [(s - 1).contiguous() for s in wl.seq_lens]
    q_draft = [wl.draft_q(j) for j in range(gamma)]
    sel = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
    nsel = torch.empty((B,), dtype=torch.int32, device=dev)
    sel_r = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
    nsel_r = torch.empty((B,), dtype=torch.int32, device=dev)
    d_out = torch.empty((gamma, B, Hq, D), dtype=torch.bfloat16, device=dev)
    v_out = torch.empty((B, gamma + 1, Hq, D), dtype=torch.bfloat16, device=dev)
    ws_sel = torch.empty(max(1, s3r.page_select_workspace(kv, budget)), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(1, s3r.attn_workspace(kv, 1, k)), dtype=torch.uint8, device=dev)
    ws_step = torch.empty(max(1, s3r.sparse_draft_step_workspace(kv, budget)), dtype=torch.uint8,
                          device=dev)
    ws_v = torch.empty(max(1, s3r.attn_workspace(kv, gamma + 1, wl.max_pages)), dtype=torch.uint8,
                       device=dev)
    ws_s = torch.empty(max(1, s3r.spec_sample_workspace(B, gamma, V)), dtype=torch.uint8, device=dev)
    out_tok = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    n_acc = torch.empty((B,), dtype=torch.int32, device=dev)
    # The drafter's own tokens: each sequence's gamma draft rows sampled by the
    # library (the Philox stream the drafter owns), as a drafter would.
    draft_tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    ws_draw = torch.empty(max(1, s3r.draft_sample_workspace(B, gamma, V)), dtype=torch.uint8, device=dev)
    ws_alpha = torch.empty(max(1, s3r.acceptance_rate_workspace(B, gamma, V)), dtype=torch.uint8,
                           device=dev)
    alpha = torch.empty((B, gamma), dtype=torch.float64, device=dev)

    def draft_draws(offset=0):
        s3r.draft_sample(wl.draft_logits, T, 0, offset, tokens=draft_tokens, workspace=ws_draw)

    def acceptance():
        s3r.acceptance_rate(wl.draft_logits, wl.target_logits, T, alpha=alpha, workspace=ws_alpha)

    draft_draws(0)

    def draft_step(j):
        kv.set_seq_lens(wl.seq_lens[j])
        s3r.sparse_draft_step(kv, bounds, q_draft[j], budget, scale, refresh_from=first_pos[j],
                              selected=sel, num_selected=nsel, out=d_out[j], workspace=ws_step)

    def verify():
        kv.set_seq_lens(wl.seq_lens[gamma])
        s3r.dense_verify_attn(kv, wl.q_verify, scale, out=v_out, workspace=ws_v)

    def sample(offset):
        s3r.spec_sample(wl.draft_logits, wl.target_logits, draft_tokens, T, 0, offset,
                        out_tokens=out_tok, num_accepted=n_acc, workspace=ws_s)

    def one_round(offset=0):
        for j in range(gamma):
            draft_step(j)
        verify()
        sample(offset)

    def one_round_select_once(offset=0):
        kv.set_seq_lens(wl.seq_lens[0])
        s3r.sparse_draft_round(kv, bounds, q_draft[0], budget, gamma, scale,
                               refresh_from=first_pos[0], selected=sel_r, num_selected=nsel_r,
                               out=d_out[0], workspace=ws_step)
        for j in range(1, gamma):
            kv.set_seq_lens(wl.seq_lens[j])
            s3r.sparse_draft_attn(kv, q_draft[j], sel_r, scale, out=d_out[j], workspace=ws_d)
        verify()
        sample(offset)

    # The one-layer autoregressive step: one query at position L-1 over all L tokens.
    q_dense = wl.q_verify[:, :1].contiguous()
    o_dense = torch.empty((B, 1, Hq, D), dtype=torch.bfloat16, device=dev)
    ws_dense = torch.empty(max(1, s3r.attn_workspace(kv, 1, wl.max_pages)), dtype=torch.uint8,
                           device=dev)

    def dense_decode(offset=0):
        kv.set_seq_lens(wl.seq_lens[0])
        s3r.dense_verify_attn(kv, q_dense, scale, out=o_dense, workspace=ws_dense)

    def accept_stats():
        """Mean accepted drafts per sequence and committed tokens per round, over 8 offsets."""
        acc = []
        for off in range(8):
            sample(off)
            acc.append(n_acc.clone())
        torch.cuda.synchronize()
        acc = torch.stack(acc).float()
        return float(acc.mean()), float((acc + 1).sum(dim=1).mean())

    return types.SimpleNamespace(**locals())


def make_runner(fn, graphed, keep):
    """A replay of fn(0) captured into a HIP graph (kept alive in `keep`), or fn itself."""
    import torch
    if not graphed:
        return lambda: fn(0)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        fn(0)
    keep.append(g)
    return g.replay


def time_runner(runner, steps, warmup):
    """Mean ms per call of `steps` back-to-back calls, synchronised on both sides."""
    import torch
    for _ in range(max(1, warmup)):
        runner()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        runner()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def main():
    args = parse()
    if args.gpus != 1:
        sys.exit(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
                 "(the S3R hot path shards by sequence, with no exchange between GPUs)")
    if args.sweep:
        return sweep(args)
    if args.fidelity:
        return fidelity(args)
    if args.shrink:
        return shrink(args)

    import torch

    import self_sparse_speculative_paged_amd as s3r

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R = build_round(args.config, dev, seed=0)
    wl, cfg, kv, bounds = R.wl, R.cfg, R.kv, R.bounds
    B, Hq, Hkv, D, P, gamma, V = R.B, R.Hq, R.Hkv, R.D, R.P, R.gamma, R.V
    budget, scale, ctx = R.budget, R.scale, R.ctx

    # eager warm-up, and the accepted-length statistics over several Philox offsets
    for w in range(max(1, args.warmup)):
        R.one_round(w)
    mean_acc, mean_committed = R.accept_stats()

    graphs = []
    ms = time_runner(make_runner(R.one_round, not args.no_graph, graphs), args.steps, args.warmup)
    ms_once = time_runner(make_runner(R.one_round_select_once, not args.no_graph, graphs),
                          args.steps, args.warmup)

    # Per-launch time of each entry point: the call captured alone into a HIP
    # graph and replayed back to back between two events on the launch stream
    # (eager calls with --no-graph), so host launch latency stays out of it.
    def time_call(fn, reps):
        return 1e3 * time_runner(make_runner(lambda _off: fn(), not args.no_graph, graphs), reps,
                                 args.warmup)

    reps = max(5, args.steps)
    kv.set_seq_lens(wl.seq_lens[0])
    t_select = time_call(lambda: s3r.page_select(kv, bounds, R.q_draft[0], budget, scale, R.sel,
                                                 R.nsel, workspace=R.ws_sel), reps)
    t_draft = time_call(lambda: s3r.sparse_draft_attn(kv, R.q_draft[0], R.sel, scale,
                                                      out=R.d_out[0], workspace=R.ws_d), reps)
    t_bounds = time_call(lambda: s3r.page_bounds_update(kv, bounds, first_pos=R.first_pos[0],
                                                        max_pages_touched=1), reps)
    t_step = time_call(lambda: s3r.sparse_draft_step(kv, bounds, R.q_draft[0], budget, scale,
                                                     refresh_from=R.first_pos[0], selected=R.sel,
                                                     num_selected=R.nsel, out=R.d_out[0],
                                                     workspace=R.ws_step), reps)
    kv.set_seq_lens(wl.seq_lens[gamma])
    t_verify = time_call(lambda: s3r.dense_verify_attn(kv, wl.q_verify, scale, out=R.v_out,
                                                       workspace=R.ws_v), reps)
    t_sample = time_call(lambda: R.sample(0), reps)
    t_draw = time_call(lambda: R.draft_draws(0), reps)
    t_alpha = time_call(R.acceptance, reps)
    R.acceptance()
    mean_alpha = float(R.alpha.mean())
    # KV commit of a verify's gamma+1 rows at the round's positions (last: it rewrites them).
    g = torch.Generator(device=dev).manual_seed(1)
    k_new = torch.randn((B, gamma + 1, Hkv, D), device=dev, generator=g).to(wl.k_pool.dtype)
    v_new = torch.randn((B, gamma + 1, Hkv, D), device=dev, generator=g).to(wl.k_pool.dtype)
    kv.set_seq_lens(wl.seq_lens[gamma])
    t_commit = time_call(lambda: s3r.kv_commit(kv, k_new, v_new, R.first_pos[0], bounds), reps)

    parts = step_bytes(cfg, ctx)
    total_bytes = sum(parts.values())
    parts_once = step_bytes(cfg, ctx, select_once=True)
    gbs = total_bytes / (ms * 1e-3) / 1e9
    verify_gbs = parts["verify"] / (t_verify * 1e-6) / 1e9
    verify_flops = verify_algorithmic_flops(cfg, ctx)
    per_step_draft = parts["draft"] / gamma
    draft_gbs = per_step_draft / (t_draft * 1e-6) / 1e9
    dv_us = gamma * t_draft + t_verify
    dv_gbs = (parts["draft"] + parts["verify"]) / (dv_us * 1e-6) / 1e9

    traffic = read_counter_traffic(args.config)
    mfma = read_counter_mfma(args.config)
    # The verify call is one kernel when its splits merge inside the workgroup
    # (no workspace); otherwise a split combine and, on ragged batches, the
    # longest-first ordering launch with it.
    verify_label = ("dense_verify_attn: one attn_bf16_kernel launch, splits merged in the workgroup"
                    if s3r.attn_workspace(kv, gamma + 1, wl.max_pages) == 0 else
                    "dense_verify_attn: attn_bf16_kernel with its split combine / ordering launches")
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 KV/Q, N(0,2)+noise fp32 logits)",
        "config": {"workload": f"{args.config}_layer", "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "context": ctx[0] if len(set(ctx)) == 1 else "ragged",
                   "page": P, "budget_tokens": budget, "gamma": gamma, "vocab": V,
                   "graph": not args.no_graph},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "accepted_tokens_per_s": round(mean_committed / (ms * 1e-3), 1),
        "mean_accepted_per_seq": round(mean_acc, 3),
        "draft_verify_kv_gbs": round(dv_gbs, 1),
        "draft_kv_gbs": round(draft_gbs, 1),
        "verify_kv_gbs": round(verify_gbs, 1),
        "step_bytes": {k2: int(v2) for k2, v2 in parts.items()},
        "launch_us": {"page_bounds_update": round(t_bounds, 2), "page_select": round(t_select, 2),
                      "sparse_draft_attn": round(t_draft, 2), "sparse_draft_step": round(t_step, 2),
                      "dense_verify_attn": round(t_verify, 2), "spec_sample": round(t_sample, 2),
                      "kv_commit": round(t_commit, 2), "draft_sample": round(t_draw, 2),
                      "acceptance_rate": round(t_alpha, 2)},
        "mean_alpha": round(mean_alpha, 4),
        "select_once": {
            "ms_per_step": round(ms_once, 4),
            "value": round(sum(parts_once.values()) / (ms_once * 1e-3) / 1e9, 1),
            "accepted_tokens_per_s": round(mean_committed / (ms_once * 1e-3), 1),
            "step_bytes": int(sum(parts_once.values())),
        },
        "roofline": {"kernel": verify_label,
                     "bound": "hbm", "achieved": round(verify_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(verify_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        # MFMA use of the same verify launch: algorithmic flops are 4 per
        # (query row, visible token, d); the matrix cores also run the padding
        # of the rows to 16-row blocks and P's second (lo) bf16 part.
        "verify_mfma": {
            "algorithmic_flops_per_launch": verify_flops,
            "algorithmic_tflops": round(verify_flops / (t_verify * 1e-6) / 1e12, 1),
            "mfma_flops_per_launch": mfma[1] if mfma else None,
            "mfma_tflops": round(mfma[1] / (t_verify * 1e-6) / 1e12, 1) if mfma else None,
            "peak_tflops_bf16": 2500.0,
            "mfma_busy_pct": mfma[0] if mfma else None,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, cfg, args.cpu_seconds)
    if not args.no_configs:
        # every other workload, timed the same way (the headline's buffers freed first)
        del R, wl, kv, bounds, graphs
        torch.cuda.empty_cache()
        result["configs"] = other_configs(args)
    print(json.dumps(result), flush=True)


def ragged_subset(n, seed=0):
    """The n longest sequences of the ragged long-tail draw, in their original
    order: the batch as it drains (short rollouts finish first)."""
    import torch

    from s3r_inputs import CONFIGS, ragged_lengths
    full = ragged_lengths(CONFIGS["ragged"]["B"], seed=seed)
    keep = torch.argsort(full, descending=True, stable=True)[:n].sort().values
    return [int(full[i]) for i in keep]


def config_summary(config, args, label, **overrides):
    """One workload's round (graph replay), its verify and draft-step launches,
    and its committed tokens per second, as a dict for the bench line."""
    import torch

    import self_sparse_speculative_paged_amd as s3r

    dev = torch.device("cuda:0")
    R = build_round(config, dev, seed=0, **overrides)
    for w in range(max(1, args.warmup)):
        R.one_round(w)
    mean_acc, committed = R.accept_stats()
    graphs = []
    ms = time_runner(make_runner(R.one_round, True, graphs), args.steps, args.warmup)
    ms_once = time_runner(make_runner(R.one_round_select_once, True, graphs), args.steps, args.warmup)

    def time_call(fn):
        return 1e3 * time_runner(make_runner(lambda _off: fn(), True, graphs), max(5, args.steps), args.warmup)

    R.kv.set_seq_lens(R.wl.seq_lens[0])
    t_step = time_call(lambda: s3r.sparse_draft_step(R.kv, R.bounds, R.q_draft[0], R.budget, R.scale,
                                                     refresh_from=R.first_pos[0], selected=R.sel,
                                                     num_selected=R.nsel, out=R.d_out[0], workspace=R.ws_step))
    R.kv.set_seq_lens(R.wl.seq_lens[R.gamma])
    t_verify = time_call(lambda: s3r.dense_verify_attn(R.kv, R.wl.q_verify, R.scale, out=R.v_out,
                                                       workspace=R.ws_v))
    t_sample = time_call(lambda: R.sample(0))
    parts = step_bytes(R.cfg, R.ctx)
    total = sum(parts.values())
    out = {
        "workload": label, "batch": R.B, "gamma": R.gamma, "budget_tokens": R.budget,
        "context": R.ctx[0] if len(set(R.ctx)) == 1 else {"min": min(R.ctx), "max": max(R.ctx),
                                                           "mean": round(sum(R.ctx) / len(R.ctx))},
        "round_ms": round(ms, 4), "value_gbs": round(total / (ms * 1e-3) / 1e9, 1),
        "pct_hbm_peak": round(100 * total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "accepted_tokens_per_s": round(committed / (ms * 1e-3), 1),
        "mean_accepted_per_seq": round(mean_acc, 3),
        "verify_us": round(t_verify, 2),
        "verify_pct_hbm_peak": round(100 * parts["verify"] / (t_verify * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
        "draft_step_us": round(t_step, 2),
        "draft_step_pct_hbm_peak": round(
            100 * (parts["draft"] + parts["select"] + parts["bounds"]) / R.gamma / (t_step * 1e-6) / 1e9
            / HBM_PEAK_GBS, 2),
        "spec_sample_us": round(t_sample, 2),
        "select_once_round_ms": round(ms_once, 4),
        "round_bytes": int(total),
    }
    del R, graphs
    torch.cuda.empty_cache()
    return out


def other_configs(args):
    """The bench line's other workloads: the Qwen3-1.7B-shaped layer, the
    aggressive budget (the whole select -> draft -> verify -> sample chain per
    round), and the ragged long tail at 128 sequences and as it drains to 64,
    16 and 8."""
    res = {"qwen3_1p7b": config_summary("qwen3_1p7b", args, "qwen3_1p7b_layer"),
           "aggressive": config_summary("aggressive", args, "aggressive_layer")}
    for n in (128, 64, 16, 8):
        res[f"ragged_{n}"] = config_summary("ragged", args, f"ragged_long_tail_{n}", B=n, ctx=ragged_subset(n))
    return res


FIDELITY_BUDGETS = (256, 512, 1024, 2048, 4096)


def fidelity(args):
    """Direct sparse sampling against S3R, per budget, through a toy head.

    A fixed random head W [32768][Hq*D] maps the dense decode output at the
    step-0 query to the dense policy's logits (p) and the sparse draft output
    to the sparse policy's logits (q), scaled per sequence so the dense logits
    have sd 2 (the workloads' draft-logit sd): W and the scaling are the
    harness's stand-in for a model, and every quantity of the method comes
    from the library. Direct sparse sampling draws from q (s3r_draft_sample):
    each token is TV(p, q) = 1 - alpha away from the dense policy, with
    alpha = sum min(p, q) from s3r_acceptance_rate. S3R draws from p exactly
    and accepts a draft with probability alpha, which s3r_spec_sample measures
    over 64 rounds of one draft each."""
    import torch

    import self_sparse_speculative_paged_amd as s3r
    from s3r_inputs import make_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = make_workload(args.config, device=dev, seed=0, with_logits=False)
    cfg = wl.cfg
    B, Hq, Hkv, D, P, gamma = (cfg[k] for k in ("B", "Hq", "Hkv", "D", "P", "gamma"))
    scale = 1.0 / math.sqrt(D)
    V_TOY = 32768
    W = torch.randn((V_TOY, Hq * D), generator=torch.Generator(device=dev).manual_seed(1), device=dev)
    kv = s3r.PagedKVCache(wl.k_pool, wl.v_pool, wl.page_table, wl.seq_lens[0], Hq)
    q0 = wl.draft_q(0)
    o_dense = s3r.dense_verify_attn(kv, q0[:, None].contiguous(), scale)[:, 0].reshape(B, Hq * D)
    z_dense = o_dense @ W.t()
    c = 2.0 / z_dense.std(dim=1, keepdim=True)
    target = torch.stack([c * z_dense, c * z_dense], dim=1).contiguous()  # the row, and a bonus row
    bounds = torch.empty((wl.k_pool.shape[0], Hkv, 2, D), dtype=wl.k_pool.dtype, device=dev)
    s3r.page_bounds_update(kv, bounds)
    for budget in FIDELITY_BUDGETS:
        sel, _ = s3r.page_select(kv, bounds, q0, budget, scale)
        o_sparse = s3r.sparse_draft_attn(kv, q0, sel, scale).reshape(B, Hq * D)
        draft = (c * (o_sparse @ W.t()))[:, None].contiguous()
        alpha = s3r.acceptance_rate(draft, target, 1.0)[:, 0]
        tv = 1.0 - alpha
        acc = []
        for off in range(64):
            x = s3r.draft_sample(draft, 1.0, budget, off)
            _, n = s3r.spec_sample(draft, target, x, 1.0, budget, off)
            acc.append(n.double())
        acc = torch.stack(acc)
        torch.cuda.synchronize()
        print(json.dumps({
            "fidelity": {"workload": f"{args.config}_layer", "budget_tokens": budget, "pages": budget // P,
                         "draft_step": 0, "toy_vocab": V_TOY},
            "tv_direct_sparse": {"mean": round(float(tv.mean()), 4),
                                 "p10": round(float(tv.quantile(0.1)), 4),
                                 "max": round(float(tv.max()), 4)},
            "alpha": round(float(alpha.mean()), 4),
            "s3r_measured_acceptance": round(float(acc.mean()), 4),
            "s3r_acceptance_sd": round(float(acc.mean(0).std() / math.sqrt(len(acc))), 4),
        }), flush=True)


SWEEP_CONTEXTS = (8192, 32768)
SWEEP_GAMMAS = (2, 4, 8)
SWEEP_NOISE = (0.5, 1.35)      # target-logit noise: per-token acceptance about 0.8 and 0.5
SWEEP_BUDGETS = (512, 2048)


def sweep(args):
    """Speedup condition over context x gamma x acceptance x budget (8B heads, batch 32)."""
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for L in SWEEP_CONTEXTS:
        for gamma in SWEEP_GAMMAS:
            for noise in SWEEP_NOISE:
                for budget in SWEEP_BUDGETS:
                    R = build_round("qwen3_8b", dev, seed=0, L=L, gamma=gamma, noise_sd=noise,
                                    budget=budget)
                    mean_acc, mean_committed = R.accept_stats()
                    E = mean_committed / R.B
                    graphs = []
                    ms = time_runner(make_runner(R.one_round, True, graphs), args.steps, args.warmup)
                    ms_once = time_runner(make_runner(R.one_round_select_once, True, graphs),
                                          args.steps, args.warmup)
                    ms_dense = time_runner(make_runner(R.dense_decode, True, graphs), args.steps,
                                           args.warmup)
                    kv_tok = 2 * R.Hkv * R.D * 2
                    dense_bytes = R.B * L * kv_tok
                    round_bytes = sum(step_bytes(R.cfg, R.ctx).values())
                    once_bytes = sum(step_bytes(R.cfg, R.ctx, select_once=True).values())
                    print(json.dumps({
                        "sweep_point": {"context": L, "gamma": gamma, "budget_tokens": budget,
                                        "target_noise_sd": noise},
                        "mean_accepted": round(mean_acc, 3), "committed_per_round": round(E, 3),
                        "round_ms": round(ms, 4), "round_select_once_ms": round(ms_once, 4),
                        "dense_decode_ms": round(ms_dense, 4),
                        "speedup": round(E * ms_dense / ms, 3),
                        "speedup_select_once": round(E * ms_dense / ms_once, 3),
                        "speedup_bytes": round(E * dense_bytes / round_bytes, 3),
                        "speedup_bytes_select_once": round(E * dense_bytes / once_bytes, 3),
                        "round_gbs": round(round_bytes / (ms * 1e-3) / 1e9, 1),
                        "dense_gbs": round(dense_bytes / (ms_dense * 1e-3) / 1e9, 1),
                    }), flush=True)
                    del R, graphs
                    torch.cuda.empty_cache()


def shrink(args):
    """The ragged long-tail batch as it drains. Short rollouts finish first, so
    the round runs on the longest 128, 64, 16 and 8 sequences of one lognormal
    draw, kept in their original order, each on a fresh seeded workload. One
    JSON line per active batch size."""
    import torch

    from s3r_inputs import CONFIGS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for n in CONFIGS["ragged"]["shrink"]:
        ctx = ragged_subset(n)
        R = build_round("ragged", dev, seed=0, B=n, ctx=ctx)
        graphs = []
        ms = time_runner(make_runner(R.one_round, True, graphs), args.steps, args.warmup)
        ms_once = time_runner(make_runner(R.one_round_select_once, True, graphs), args.steps, args.warmup)
        parts = step_bytes(R.cfg, R.ctx)
        once = sum(step_bytes(R.cfg, R.ctx, select_once=True).values())
        gbs = sum(parts.values()) / (ms * 1e-3) / 1e9
        _, committed = R.accept_stats()
        print(json.dumps({
            "shrink_point": {"active_batch": n, "context_min": min(ctx), "context_median": sorted(ctx)[n // 2],
                             "context_max": max(ctx), "kv_gb": round(parts["verify"] / 1e9, 3)},
            "round_ms": round(ms, 4), "value_gbs": round(gbs, 1),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "accepted_tokens_per_s": round(committed / (ms * 1e-3), 1),
            "round_select_once_ms": round(ms_once, 4),
            "select_once_gbs": round(once / (ms_once * 1e-3) / 1e9, 1),
        }), flush=True)
        del R, graphs
        torch.cuda.empty_cache()


def _profile_fields(name):
    """The `key: value` fields of a committed rocprofv3 summary under profiles/,
    or None when it is missing or was taken on a different attention kernel
    source (its recorded hash no longer matches)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    src = os.path.join(ROOT, "self_sparse_speculative_paged_amd", "csrc", "s3r_attn.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    return fields if fields.get("kernel_source_sha256_16") == digest else None


def read_counter_traffic(config):
    """HBM bytes per verify launch from the committed counter summary, or None."""
    fields = _profile_fields(f"counters_dense_verify_{config}.txt")
    try:
        return int(fields["hbm_bytes_per_launch"]) if fields else None
    except (KeyError, ValueError):
        return None


def read_counter_mfma(config):
    """(MFMA busy %, bf16 MFMA flops) per verify launch from the committed
    counter summary, or None."""
    fields = _profile_fields(f"counters_mfma_dense_verify_{config}.txt")
    try:
        return (float(fields["mfma_util_pct"]), int(fields["mfma_flops_bf16_per_launch"])) if fields else None
    except (KeyError, ValueError):
        return None


def _oracle_worker_init():
    """Worker start-up: the oracle's imports, single-threaded BLAS."""
    import numpy  # noqa: F401
    import threadpoolctl  # noqa: F401

    import oracle  # noqa: F401


def _oracle_slice(task):
    """One (sequence, kv head) slice of the round through the oracle, in a worker
    process. The slice's pages are gathered from the pools in shared memory
    and upcast to fp64 (set-up, untimed). Returns (bytes, seconds) of
    `_run_oracle_slice`."""
    from multiprocessing import shared_memory

    import numpy as np

    (names, shapes, bf16, idx, h, L, cfg, q_ver, logits) = task
    arrays = []
    for name, shape in zip(names, shapes):
        shm = shared_memory.SharedMemory(name=name)
        try:
            pool = np.ndarray(shape, dtype=np.uint16 if bf16 else np.float32, buffer=shm.buf)
            part = pool[idx, h:h + 1]
            if bf16:
                part = (part.astype(np.uint32) << 16).view(np.float32)
            arrays.append(part.astype(np.float64))
            del pool, part
        finally:
            shm.close()
    return _run_oracle_slice(arrays[0], arrays[1], bf16, L, cfg, q_ver, logits)


def _run_oracle_slice(K, Vv, bf16, L, cfg, q_ver, logits):
    """The timed part of one slice: the slice's page bounds (untimed set-up),
    then gamma x (page_select + sparse draft), the dense verify and, when
    `logits` is given, the sequence's spec_sample, single-threaded. K and Vv
    hold the slice's pages in order, fp64. Returns (bytes, seconds)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    P, D, gamma, V = (cfg[k] for k in ("P", "D", "gamma", "V"))
    esz = 2 if bf16 else 4
    scale = 1.0 / math.sqrt(D)
    k = cfg["budget"] // P
    pt = np.arange(K.shape[0], dtype=np.int64)[None, :]
    bounds = oracle.page_bounds(K, pt, np.array([L + gamma]))
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        for j in range(gamma):
            lens = np.array([L + j])
            qd = q_ver[:, j]
            sel, _, _ = oracle.page_select(bounds, qd, pt, lens, cfg["budget"], scale, P)
            oracle.sparse_draft_attn(qd, K, Vv, pt, lens, sel, scale)
            nj = -(-(L + j) // P)
            done += nj * 2 * D * esz + min(k, nj) * P * 2 * D * esz
        oracle.dense_verify_attn(q_ver, K, Vv, pt, np.array([L + gamma]), scale)
        done += (L + gamma) * 2 * D * esz
        if logits is not None:
            oracle.spec_sample(logits[0], logits[1], logits[2], cfg["temperature"], 0, 0)
            done += (2 * gamma + 1) * V * 4
    return done, time.perf_counter() - t0


def _shm_free_bytes():
    try:
        st = os.statvfs("/dev/shm")
        return st.f_bavail * st.f_frsize
    except OSError:
        return 0


def cpu_baseline(wl, cfg, budget_s):
    """The oracle, as it stands, on the round's (sequence, kv head) slices, one
    slice per task over a pool of worker processes, one per host core of the
    GPU's share (at most 16). Slices are handed out until about `budget_s`
    seconds of wall time have passed (the whole round normally fits). The
    value is the algorithmic bytes of the slices done over the wall time of
    the pool phase. The pools sit in host shared memory, copied once from the
    device before the clock starts. The wall time includes each worker's
    gather and upcast of its slice.

    Where /dev/shm cannot hold both pools (with a margin), the slices run in
    this process instead, one core, each slice gathered from the device
    before its clock starts; the value is then the bytes over the summed
    slice times, and the sample says so."""
    import numpy as np
    import torch

    P, Hkv, Hq, gamma = (cfg[k] for k in ("P", "Hkv", "Hq", "gamma"))
    G = Hq // Hkv
    bf16 = cfg["kv_dtype"] == "bf16"

    def slices():
        for b in range(cfg["B"]):
            L = int(wl.ctx[b])
            idx = wl.page_table[b, :-(-(L + gamma) // P)].long()
            logits = (wl.draft_logits[b:b + 1].to("cpu", torch.float64).numpy(),
                      wl.target_logits[b:b + 1].to("cpu", torch.float64).numpy(),
                      wl.draft_tokens[b:b + 1].cpu().numpy())
            for h in range(Hkv):
                q = wl.q_verify[b:b + 1, :, h * G:(h + 1) * G].to("cpu", torch.float64).numpy()
                yield idx, h, L, q, logits if h == 0 else None

    what = (f"each: {gamma} draft steps (page_select + sparse attention), dense verify of {gamma + 1} "
            f"queries x {G} heads over the full context, plus spec_sample (vocab {cfg['V']}) "
            f"once per sequence; fp64 NumPy")
    need = sum(t.numel() * t.element_size() for t in (wl.k_pool, wl.v_pool))
    if _shm_free_bytes() < need + need // 10 + (1 << 30):
        total, spent, n = 0, 0.0, 0
        t0 = time.perf_counter()
        for idx, h, L, q, logits in slices():
            if time.perf_counter() - t0 >= budget_s:
                break
            K, Vv = (t[idx, h:h + 1].to("cpu", torch.float64).numpy() for t in (wl.k_pool, wl.v_pool))
            done, sec = _run_oracle_slice(K, Vv, bf16, L, cfg, q, logits)
            total, spent, n = total + done, spent + sec, n + 1
        return {"value": round(total / spent / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "bytes": total, "seconds": round(spent, 2),
                "sample": f"{n} of the {cfg['B'] * Hkv} (sequence, kv head) slices of the round, {what}; "
                          f"one process, 1 thread (/dev/shm too small for the pooled run)"}

    import multiprocessing as mp
    from multiprocessing import shared_memory

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    shms, names, shapes = [], [], []
    try:
        for t in (wl.k_pool, wl.v_pool):
            host_dt, dev_view = (np.uint16, t.view(torch.int16)) if bf16 else (np.float32, t)
            shm = shared_memory.SharedMemory(create=True, size=t.numel() * t.element_size())
            shms.append(shm)
            arr = np.ndarray(tuple(t.shape), dtype=host_dt, buffer=shm.buf)
            torch.from_numpy(arr.view(np.int16) if bf16 else arr).copy_(dev_view)
            del arr
            names.append(shm.name)
            shapes.append(tuple(t.shape))
        ctx = mp.get_context("spawn")  # the workers never touch the GPU
        with ctx.Pool(workers, initializer=_oracle_worker_init) as pool:
            pool.map(abs, range(4 * workers))  # every worker started and initialised
            pending, total, n = [], 0, 0
            t0 = time.perf_counter()
            for idx, h, L, q, logits in slices():
                if time.perf_counter() - t0 >= budget_s:
                    break
                task = (names, shapes, bf16, idx.cpu().numpy(), h, L, cfg, q, logits)
                pending.append(pool.apply_async(_oracle_slice, (task,)))
                while len(pending) >= 2 * workers:  # bounded host memory in flight
                    total += pending.pop(0).get()[0]
                    n += 1
            for r in pending:
                total += r.get()[0]
                n += 1
            wall = time.perf_counter() - t0
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    return {"value": round(total / wall / 1e9, 6), "unit": "GB/s", "cores": workers,
            "kind": "oracle", "bytes": total, "seconds": round(wall, 2),
            "sample": f"{n} of the {cfg['B'] * Hkv} (sequence, kv head) slices of the round, {what}, "
                      f"{workers} worker processes, 1 thread each"}


if __name__ == "__main__":
    main()

"""Per-slice oracle checks of the full-size workloads, in a pool of spawned
worker processes that never touch the GPU.

Test infrastructure: the K/V pools are copied once from the device into host
shared memory (bf16 kept as its 16-bit pattern); each task names one
(sequence, kv head) slice by its page ids and carries the GPU's outputs for
that slice. A worker gathers the slice's pages, upcasts them exactly to fp64
(slot order kept, so the slice's page table is 0..n-1) and calls a check
function of this module, which runs the oracle and returns a list of error
strings. Data movement only here; the arithmetic is the oracle's.
"""
import math
import os
import time

import numpy as np

import oracle
from tests.parity import check_pages

_POOLS = {}


def _attach(names, shapes, bf16):
    from multiprocessing import shared_memory
    key = tuple(names)
    if key not in _POOLS:
        shms = [shared_memory.SharedMemory(name=n) for n in names]
        dt = np.uint16 if bf16 else np.float32
        _POOLS[key] = (shms, [np.ndarray(s, dtype=dt, buffer=m.buf) for s, m in zip(shapes, shms)])
    return _POOLS[key][1]


def _upcast(part, bf16):
    if bf16:
        part = (part.astype(np.uint32) << 16).view(np.float32)
    return part.astype(np.float64)


def _worker_init():
    import threadpoolctl
    threadpoolctl.threadpool_limits(1)


def _run_task(args):
    names, shapes, bf16, fn, task = args
    k_pool, v_pool = _attach(names, shapes, bf16)
    idx, h = task["idx"], task["h"]
    K = _upcast(k_pool[idx, h:h + 1], bf16)
    V = _upcast(v_pool[idx, h:h + 1], bf16)
    try:
        return task["key"], globals()[fn](K, V, task)
    except Exception as e:  # a crash in a check is a failure of that slice
        return task["key"], [f"{type(e).__name__}: {e}"]


def _shm_free():
    try:
        st = os.statvfs("/dev/shm")
        return st.f_bavail * st.f_frsize
    except OSError:
        return 0


def pool_fits(k_pool, v_pool):
    need = sum(t.numel() * t.element_size() for t in (k_pool, v_pool))
    return _shm_free() >= need + need // 10 + (1 << 30)


def run(k_pool, v_pool, fn, tasks, workers=None):
    """Run check `fn` (a name in this module) on every task; returns
    {key: [errors]} for the slices that failed and the wall time."""
    import multiprocessing as mp
    from multiprocessing import shared_memory

    import torch

    bf16 = k_pool.dtype == torch.bfloat16
    workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    shms, names, shapes = [], [], []
    t0 = time.perf_counter()
    try:
        for t in (k_pool, v_pool):
            shm = shared_memory.SharedMemory(create=True, size=t.numel() * t.element_size())
            shms.append(shm)
            host_dt, dev_view = (np.uint16, t.view(torch.int16)) if bf16 else (np.float32, t)
            arr = np.ndarray(tuple(t.shape), dtype=host_dt, buffer=shm.buf)
            torch.from_numpy(arr.view(np.int16) if bf16 else arr).copy_(dev_view)
            del arr
            names.append(shm.name)
            shapes.append(tuple(t.shape))
        ctx = mp.get_context("spawn")
        failed = {}
        with ctx.Pool(workers, initializer=_worker_init) as pool:
            jobs = [(names, shapes, bf16, fn, task) for task in tasks]
            for key, errs in pool.imap_unordered(_run_task, jobs, chunksize=1):
                if errs:
                    failed[key] = errs
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    return failed, time.perf_counter() - t0


def run_local(k_pool, v_pool, fn, tasks):
    """The same checks in this process (no shared memory), for hosts whose
    /dev/shm cannot hold the pools."""
    import torch
    bf16 = k_pool.dtype == torch.bfloat16
    failed = {}
    for task in tasks:
        idx = torch.as_tensor(task["idx"], dtype=torch.long, device=k_pool.device)
        h = task["h"]
        K = k_pool.index_select(0, idx)[:, h:h + 1].to("cpu", torch.float64).numpy()
        V = v_pool.index_select(0, idx)[:, h:h + 1].to("cpu", torch.float64).numpy()
        errs = globals()[fn](K, V, task)
        if errs:
            failed[task["key"]] = errs
    return failed


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_round_slice(K, V, t):
    """One (sequence, kv head) slice of a full-size round, against the oracle:
    the draft step's bounds (exact), selection (1e-4 tie window) and sparse
    attention (1e-2), the dense verify of gamma + 1 queries (1e-2), and the
    once-per-round selection with its reuse at the round's last draft step."""
    errs = []
    c = t["cfg"]
    P, gamma, budget, L = c["P"], c["gamma"], c["budget"], t["L"]
    k = budget // P
    scale = 1.0 / math.sqrt(c["D"])
    n = K.shape[0]
    pt = np.arange(n, dtype=np.int64)[None, :]
    lens = np.array([L])
    rb = oracle.page_bounds(K, pt, lens)
    n0 = oracle.n_pages(L, P)
    got_b = _bf16_to_f64(t["bounds"]) if t["bf16"] else t["bounds"]
    if not np.array_equal(got_b[:n0], rb[:n0, 0]):  # [page][min|max][d] of kv head h
        errs.append("bounds")
    q0 = t["q0"][None]
    rsel, rn, rsc = oracle.page_select(rb, q0, pt, lens, budget, scale, P)
    try:
        check_pages(t["sel"][None, None], np.array([t["nsel"]]), rsel, rn, rsc, k)
    except AssertionError as e:
        errs.append(f"selection {e}")
    rd = oracle.sparse_draft_attn(q0, K, V, pt, lens, t["sel"][None, None], scale)
    err = float(np.max(np.abs(t["draft"] - rd[0])))
    if not err <= 1e-2:
        errs.append(f"draft {err}")
    rv = oracle.dense_verify_attn(t["qv"][None], K, V, pt, np.array([L + gamma]), scale)
    err = float(np.max(np.abs(t["verify"] - rv[0])))
    if not err <= 1e-2:
        errs.append(f"verify {err}")
    # once-per-round selection at step 0 (forced pages exact, the rest in the tie window)
    rr, rrn, rrsc = oracle.page_select_round(rb, q0, pt, lens, budget, gamma, scale, P)
    g = [int(x) for x in t["round_sel"] if x >= 0]
    r = [int(x) for x in rr[0, 0] if x >= 0]
    forced = oracle.round_forced_pages(L, gamma, P, t["max_pages"])
    if int(t["round_nsel"]) != int(rrn[0]) or len(g) != len(r) or not set(forced) <= set(g) or g != sorted(g):
        errs.append(f"round selection {g[:8]} {r[:8]}")
    elif g != r:
        sc = rrsc[(0, 0)]
        kth = sorted(sc.values(), reverse=True)[k - len(forced) - 1]
        if not all(j in sc and abs(sc[j] - kth) <= 1e-4 for j in set(g) ^ set(r)):
            errs.append("round selection tie window")
    rl = oracle.sparse_draft_attn(t["q_last"][None], K, V, pt, np.array([L + gamma - 1]),
                                  t["round_sel"][None, None], scale)
    err = float(np.max(np.abs(t["round_draft"] - rl[0])))
    if not err <= 1e-2:
        errs.append(f"round draft {err}")
    return errs

"""Test-side helpers: move workload tensors to the oracle's numpy fp64 form.

Pure data movement (dtype upcast, host copy, gathering a sub-pool by page
table); no arithmetic of the method lives here.
"""
import numpy as np
import torch


def f64(t):
    """Exact fp64 upcast of a bf16/fp32 tensor as a numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def i32(t):
    return t.detach().to("cpu").to(torch.int32).numpy()


def sub_pool(wl, seqs, npages=None):
    """Host fp64 copy of only the pages of `seqs`, with a page table remapped to it.

    Returns (k_pool, v_pool, page_table) where page_table has rows for every
    sequence (rows not in `seqs` point at page 0) so sequence indices keep
    their meaning.
    """
    pt = wl.page_table.to("cpu")
    B, maxp = pt.shape
    phys = []
    new_pt = np.zeros((B, maxp), dtype=np.int64)
    for b in seqs:
        n = maxp if npages is None else npages[b]
        ids = pt[b, :n]
        base = len(phys)
        phys.extend(ids.tolist())
        new_pt[b, :n] = np.arange(base, base + n)
    idx = torch.tensor(phys, dtype=torch.long, device=wl.k_pool.device)
    return f64(wl.k_pool.index_select(0, idx)), f64(wl.v_pool.index_select(0, idx)), new_pt

"""The C-ABI library loads and exports every symbol include/s3r.h declares, and
every invalid argument is rejected on the host before any HIP call (no GPU is
touched here)."""
import ctypes
import os
import re

import pytest

from self_sparse_speculative_paged_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "s3r.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(s3r_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.s3r_version() == 300
    assert lib.s3r_status_string(3) == b"S3R_ERR_WORKSPACE_TOO_SMALL"
    assert lib.s3r_status_string(99) == b"S3R_ERR_UNKNOWN"


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _kv(**kw):
    f = dict(num_seqs=2, num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
             max_pages_per_seq=8, total_pages_hint=0, kv_dtype=_lib.S3R_BF16,
             k_pool=FAKE, v_pool=FAKE, page_table=FAKE, seq_lens=FAKE, num_phys_pages=0)
    f.update(kw)
    return _lib.PagedKV(**f)


BAD_KV = [
    (dict(num_seqs=0), 1), (dict(num_q_heads=3), 1), (dict(num_kv_heads=0), 1),
    (dict(max_pages_per_seq=0), 1), (dict(total_pages_hint=-1), 1), (dict(num_phys_pages=-1), 1),
    (dict(k_pool=None), 1),
    (dict(v_pool=None), 1), (dict(page_table=None), 1), (dict(seq_lens=None), 1),
    (dict(head_dim=96), 2), (dict(page_size=32), 2), (dict(kv_dtype=7), 2),
    (dict(num_q_heads=18, num_kv_heads=2), 2),
    (dict(num_seqs=(1 << 22) + 1), 2),   # num_seqs * num_q_heads past 2^24
    (dict(num_seqs=1 << 30, num_q_heads=8, num_kv_heads=8), 2),
]


@pytest.mark.parametrize("bad,code", BAD_KV)
def test_invalid_kv_rejected_everywhere(bad, code):
    lib = _lib.load()
    kv = ctypes.byref(_kv(**bad))
    v = ctypes.c_void_p(FAKE)
    assert lib.s3r_page_bounds_update(kv, v, None, 1, None) == code
    assert lib.s3r_page_select(kv, v, v, 64, 0.1, v, v, v, 1 << 30, None) == code
    assert lib.s3r_sparse_draft_attn(kv, v, v, 4, 0.1, 0, v, v, 1 << 30, None) == code
    assert lib.s3r_dense_verify_attn(kv, v, 5, 0.1, 0, v, v, 1 << 30, None) == code
    assert lib.s3r_attn_workspace(kv, 5, 8) == 0
    assert lib.s3r_page_select_workspace(kv, 64) == 0
    assert lib.s3r_sparse_draft_step(kv, v, None, v, 64, 0.1, v, v, 0, v, v, 1 << 30, None) == code
    assert lib.s3r_sparse_draft_round(kv, v, None, v, 64, 4, 0.1, v, v, 0, v, v, 1 << 30, None) == code
    assert lib.s3r_kv_commit(kv, v, v, v, 4, v, None) == code
    assert lib.s3r_sparse_draft_step_workspace(kv, 64) == 0


def test_invalid_call_arguments():
    lib = _lib.load()
    kv = ctypes.byref(_kv())
    v = ctypes.c_void_p(FAKE)
    big = 1 << 30
    assert lib.s3r_page_bounds_update(kv, None, None, 1, None) == 1
    assert lib.s3r_page_bounds_update(kv, v, v, 0, None) == 1
    assert lib.s3r_page_select(kv, v, v, 15, 0.1, v, v, v, big, None) == 1      # budget < P
    assert lib.s3r_page_select(kv, None, v, 64, 0.1, v, v, v, big, None) == 1
    assert lib.s3r_page_select(kv, v, v, 64, float("nan"), v, v, v, big, None) == 1
    need = lib.s3r_page_select_workspace(kv, 64)
    assert need == 2 * 2 * 8 * 4
    assert lib.s3r_page_select(kv, v, v, 64, 0.1, v, v, v, need - 1, None) == 3
    assert lib.s3r_page_select(kv, v, v, 64, 0.1, v, v, None, need, None) == 1
    assert lib.s3r_sparse_draft_attn(kv, v, None, 4, 0.1, 0, v, v, big, None) == 1
    assert lib.s3r_sparse_draft_attn(kv, v, v, 0, 0.1, 0, v, v, big, None) == 1
    assert lib.s3r_sparse_draft_attn(kv, v, v, 4, 0.1, 5, v, v, big, None) == 2   # out dtype
    assert lib.s3r_dense_verify_attn(kv, v, 0, 0.1, 0, v, v, big, None) == 1
    assert lib.s3r_dense_verify_attn(kv, None, 5, 0.1, 0, v, v, big, None) == 1
    assert lib.s3r_dense_verify_attn(kv, v, 33, 0.1, 0, v, v, big, None) == 2     # 2*33 rows > 64
    kv32 = ctypes.byref(_kv(kv_dtype=_lib.S3R_F32))  # fp32 KV always merges through the workspace
    wneed = lib.s3r_attn_workspace(kv32, 5, 8)
    assert wneed > 0
    assert lib.s3r_dense_verify_attn(kv32, v, 5, 0.1, 0, v, v, wneed - 1, None) == 3
    # bf16 KV whose splits fit one workgroup merges in LDS and needs no workspace
    assert lib.s3r_attn_workspace(kv, 5, 8) == 0
    s = lib.s3r_spec_sample
    assert s(0, 4, 1024, v, v, v, 1.0, 0, 0, v, v, v, big, None) == 1
    assert s(2, 0, 1024, v, v, v, 1.0, 0, 0, v, v, v, big, None) == 1
    assert s(2, 17, 1024, v, v, v, 1.0, 0, 0, v, v, v, big, None) == 1
    assert s(2, 4, 0, v, v, v, 1.0, 0, 0, v, v, v, big, None) == 1
    assert s(2, 4, 1024, v, v, v, 0.0, 0, 0, v, v, v, big, None) == 1
    assert s(2, 4, 1024, v, v, v, float("inf"), 0, 0, v, v, v, big, None) == 1
    assert s(2, 4, 1024, None, v, v, 1.0, 0, 0, v, v, v, big, None) == 1
    sneed = lib.s3r_spec_sample_workspace(2, 4, 1024)
    assert sneed > 0 and lib.s3r_spec_sample_workspace(2, 17, 1024) == 0
    assert s(2, 4, 1024, v, v, v, 1.0, 0, 0, v, v, v, sneed - 1, None) == 3
    ds = lib.s3r_draft_sample
    assert ds(0, 4, 1024, v, 1.0, 0, 0, 0, v, v, big, None) == 1          # num_seqs
    assert ds(2, 0, 1024, v, 1.0, 0, 0, 0, v, v, big, None) == 1          # n_rows
    assert ds(2, 4, 0, v, 1.0, 0, 0, 0, v, v, big, None) == 1             # vocab
    assert ds(2, 4, 1024, v, 1.0, 0, 0, -1, v, v, big, None) == 1         # first_slot
    assert ds(2, 4, 1024, v, float("nan"), 0, 0, 0, v, v, big, None) == 1
    assert ds(2, 4, 1024, None, 1.0, 0, 0, 0, v, v, big, None) == 1
    assert ds(2, 4, 1024, v, 1.0, 0, 0, 0, None, v, big, None) == 1
    assert ds(1 << 20, 1 << 10, 1 << 20, v, 1.0, 0, 0, 0, v, v, big, None) == 2   # grid too large
    # exactly 2^31 blocks (32768 x 16 rows x 4096 chunks) is refused; one row fewer
    # passes the grid check and stops at the workspace
    assert ds(1 << 15, 16, 1 << 24, v, 1.0, 0, 0, 0, v, v, 1, None) == 2
    assert ds(1 << 15, 15, 1 << 24, v, 1.0, 0, 0, 0, v, v, 1, None) == 3
    assert s(1 << 15, 8, 1 << 24, v, v, v, 1.0, 0, 0, v, v, v, big, None) == 2   # 17 rows x 2^27 > 2^31
    dsneed = lib.s3r_draft_sample_workspace(2, 4, 1024)
    assert dsneed > 0 and lib.s3r_draft_sample_workspace(2, 0, 1024) == 0
    assert ds(2, 4, 1024, v, 1.0, 0, 0, 0, v, v, dsneed - 1, None) == 3
    assert ds(2, 4, 1024, v, 1.0, 0, 0, 0, v, ctypes.c_void_p(FAKE + 4), big, None) == 1  # workspace
    ar = lib.s3r_acceptance_rate
    assert ar(0, 4, 1024, v, v, 1.0, v, v, big, None) == 1
    assert ar(2, 0, 1024, v, v, 1.0, v, v, big, None) == 1
    assert ar(2, 4, 0, v, v, 1.0, v, v, big, None) == 1
    assert ar(2, 4, 1024, v, v, -1.0, v, v, big, None) == 1
    assert ar(2, 4, 1024, None, v, 1.0, v, v, big, None) == 1
    assert ar(2, 4, 1024, v, None, 1.0, v, v, big, None) == 1
    assert ar(2, 4, 1024, v, v, 1.0, None, v, big, None) == 1
    assert ar(2, 4, 1024, v, v, 1.0, ctypes.c_void_p(FAKE + 4), v, big, None) == 1  # alpha alignment
    assert ar(1 << 15, 8, 1 << 24, v, v, 1.0, v, v, big, None) == 2  # 16 rows x 2^27 chunks = 2^31 blocks
    arneed = lib.s3r_acceptance_rate_workspace(2, 4, 1024)
    assert arneed > 0 and lib.s3r_acceptance_rate_workspace(2, 4, 0) == 0
    assert ar(2, 4, 1024, v, v, 1.0, v, v, arneed - 1, None) == 3
    d = lib.s3r_sparse_draft_step
    assert d(kv, None, None, v, 64, 0.1, v, v, 0, v, v, big, None) == 1      # bounds
    assert d(kv, v, None, v, 15, 0.1, v, v, 0, v, v, big, None) == 1        # budget < P
    assert d(kv, v, None, v, 64, 0.1, None, v, 0, v, v, big, None) == 1     # selected
    assert d(kv, v, None, v, 64, 0.1, v, v, 7, v, v, big, None) == 2        # out dtype
    dneed = lib.s3r_sparse_draft_step_workspace(kv, 64)
    assert dneed > 0  # the page scores
    assert d(kv, v, None, v, 64, 0.1, v, v, 0, v, v, dneed - 1, None) == 3
    c = lib.s3r_kv_commit
    assert c(kv, v, v, None, 4, v, None) == 1                    # first_pos
    assert c(kv, v, v, v, -1, v, None) == 1                      # count < 0
    assert c(kv, None, v, v, 4, v, None) == 1                    # rows
    assert c(kv, ctypes.c_void_p(FAKE + 8), v, v, 4, v, None) == 1   # misaligned rows
    r = lib.s3r_sparse_draft_round
    assert r(kv, v, None, v, 64, 0, 0.1, v, v, 0, v, v, big, None) == 1      # gamma < 1
    assert r(kv, v, None, v, 64, 17, 0.1, v, v, 0, v, v, big, None) == 1     # gamma > 16
    assert r(kv, v, None, v, 31, 4, 0.1, v, v, 0, v, v, big, None) == 1      # budget < 2 pages
    assert r(kv, None, None, v, 64, 4, 0.1, v, v, 0, v, v, big, None) == 1   # bounds
    assert r(kv, v, None, v, 64, 4, 0.1, v, v, 0, v, v, dneed - 1, None) == 3


def test_split_plan_workspace_scales_with_hint():
    lib = _lib.load()
    full = lib.s3r_attn_workspace(ctypes.byref(_kv(max_pages_per_seq=4096, num_seqs=8)), 5, 4096)
    hinted = lib.s3r_attn_workspace(
        ctypes.byref(_kv(max_pages_per_seq=4096, num_seqs=8, total_pages_hint=8 * 600)), 5, 4096)
    assert hinted >= full  # a smaller average length means shorter splits, more of them


def test_drained_two_row_block_verify_takes_finer_splits():
    """A two-row-block verify over fewer than 256 (sequence, kv head) pairs whose
    page hint is under 3/4 of B * max_pages (a drained ragged batch) targets
    4096 splits instead of 1024. At 16 sequences x 8 kv heads, 4096 pages max,
    hint 33697 pages, 20 rows: 2106 pages on average over 32 splits is 66 pages a
    split, 63 splits, 16 groups of four waves; with the hint at B * max_pages the
    same batch has 512-page splits, 8 splits, 2 groups. The workspace holds one
    (rows x (D + 2)) fp32 partial per group."""
    lib = _lib.load()
    shape = dict(num_seqs=16, num_q_heads=32, num_kv_heads=8, head_dim=128, max_pages_per_seq=4096)
    partial = 20 * (128 + 2) * 4
    drained = lib.s3r_attn_workspace(ctypes.byref(_kv(total_pages_hint=33697, **shape)), 5, 4096)
    uniform = lib.s3r_attn_workspace(ctypes.byref(_kv(total_pages_hint=16 * 4096, **shape)), 5, 4096)
    assert drained == 16 * 8 * 16 * partial
    assert uniform == 16 * 8 * 2 * partial
    # 256 pairs (the Qwen3-8B batch) keep the usual target
    big = dict(shape, num_seqs=32)
    assert (lib.s3r_attn_workspace(ctypes.byref(_kv(total_pages_hint=32 * 2000, **big)), 5, 4096)
            < 32 * 8 * 16 * partial)


def test_ragged_hint_reserves_the_longest_first_order():
    """Once the page hint drops below half of B * max_pages (a ragged batch), the
    attention and draft-step workspaces also hold the sequence order: B int32,
    256-byte aligned. Hints either side of that line give the same split plan."""
    lib = _lib.load()
    B, maxp = 300, 4096
    even = ctypes.byref(_kv(max_pages_per_seq=maxp, num_seqs=B, total_pages_hint=B * maxp // 2))
    ragged = ctypes.byref(_kv(max_pages_per_seq=maxp, num_seqs=B, total_pages_hint=B * maxp // 2 - 1))
    order = (4 * B + 255) // 256 * 256
    assert lib.s3r_attn_workspace(ragged, 5, maxp) >= lib.s3r_attn_workspace(even, 5, maxp) + order
    assert (lib.s3r_sparse_draft_step_workspace(ragged, 2048)
            >= lib.s3r_sparse_draft_step_workspace(even, 2048) + order)


def test_misaligned_pointers_rejected():
    """Every 16-byte vector operand is checked on the host (INVALID_ARGUMENT)."""
    lib = _lib.load()
    v = ctypes.c_void_p(FAKE)
    m = ctypes.c_void_p(FAKE + 2)  # bf16-aligned, not 16-byte aligned
    big = 1 << 30
    kv = ctypes.byref(_kv())
    for bad in (dict(k_pool=FAKE + 2), dict(v_pool=FAKE + 8)):
        assert lib.s3r_dense_verify_attn(ctypes.byref(_kv(**bad)), v, 5, 0.1, 0, v, v, big, None) == 1
    assert lib.s3r_page_bounds_update(kv, m, None, 1, None) == 1                       # bounds
    assert lib.s3r_page_select(kv, m, v, 64, 0.1, v, v, v, big, None) == 1             # bounds
    assert lib.s3r_page_select(kv, v, m, 64, 0.1, v, v, v, big, None) == 1             # q
    assert lib.s3r_page_select(kv, v, v, 64, 0.1, v, v, m, big, None) == 1             # workspace
    assert lib.s3r_sparse_draft_attn(kv, m, v, 4, 0.1, 0, v, v, big, None) == 1       # q
    assert lib.s3r_sparse_draft_attn(kv, v, v, 4, 0.1, 0, m, v, big, None) == 1       # out
    kv32 = ctypes.byref(_kv(kv_dtype=_lib.S3R_F32))  # fp32 partials go through the workspace
    assert lib.s3r_attn_workspace(kv32, 5, 8) > 0
    assert lib.s3r_dense_verify_attn(kv32, v, 5, 0.1, 0, v, m, big, None) == 1        # workspace
    assert lib.s3r_sparse_draft_step(kv, m, None, v, 64, 0.1, v, v, 0, v, v, big, None) == 1  # bounds
    assert lib.s3r_sparse_draft_round(kv, v, None, v, 64, 4, 0.1, v, v, 0, m, v, big, None) == 1  # out
    assert lib.s3r_kv_commit(kv, v, m, v, 4, v, None) == 1                             # v_new
    assert lib.s3r_kv_commit(kv, v, v, v, 4, m, None) == 1                             # bounds
    assert lib.s3r_spec_sample(2, 4, 100, v, v, v, 1.0, 0, 0, v, v, m, big, None) == 1  # workspace


def test_binding_refuses_host_tensors():
    """The Python binding only marshals device tensors; host tensors are refused
    before the library is called."""
    import torch

    import self_sparse_speculative_paged_amd as s3r
    d = torch.zeros((2, 4, 100))
    t = torch.zeros((2, 5, 100))
    x = torch.zeros((2, 4), dtype=torch.int32)
    with pytest.raises(ValueError):
        s3r.spec_sample(d, t, x, 1.0, 0, 0)
    with pytest.raises(ValueError):
        s3r.PagedKVCache(torch.zeros((4, 2, 16, 64)), torch.zeros((4, 2, 64, 16)),
                         torch.zeros((2, 2), dtype=torch.int32), torch.zeros(2, dtype=torch.int32), 4)

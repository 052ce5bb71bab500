"""Python binding of libs3r, the S3R hot path on MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.
torch supplies device memory and the current stream. Each function checks its
tensors' device, dtype, shape and contiguity, passes raw pointers to the C ABI
and raises S3RError on a non-zero status. Outputs and workspaces may be passed
in (pre-allocated, e.g. for timing or graph capture) or are allocated here.

Entry points (same names as include/s3r.h without the prefix):
  page_bounds_update, page_select, sparse_draft_attn, sparse_draft_step (the
  three fused), sparse_draft_round (a draft step whose selection the round's
  later steps reuse), kv_commit (write new K/V rows, keep the bounds exact,
  roll back), dense_verify_attn, spec_sample, draft_sample (the drafter's own
  draws from its logits), acceptance_rate (alpha = sum min(p, q) per draft
  position), and the workspace queries.
"""
import ctypes
import functools
import threading

import torch

from . import _lib
from ._lib import PagedKV

__all__ = [
    "S3RError", "PagedKVCache", "page_bounds_update", "page_select", "sparse_draft_attn",
    "dense_verify_attn", "spec_sample", "page_select_workspace", "attn_workspace",
    "spec_sample_workspace", "version", "sparse_draft_step", "sparse_draft_step_workspace",
    "sparse_draft_round", "kv_commit", "draft_sample", "draft_sample_workspace",
    "acceptance_rate", "acceptance_rate_workspace", "spec_sample_noalloc",
]

_KV_DTYPES = {torch.float32: _lib.S3R_F32, torch.bfloat16: _lib.S3R_BF16}


class S3RError(RuntimeError):
    def __init__(self, status, where):
        lib = _lib.load()
        super().__init__(f"{where}: {lib.s3r_status_string(status).decode()} ({status})")
        self.status = status


def _check(status, where):
    if status != _lib.S3R_OK:
        raise S3RError(status, where)


_call = threading.local()  # the device of the entry-point call in progress on this thread


def _on_device(fn):
    """Runs an entry point with the device of its first argument (the KV cache,
    or the draft logits) current: the library launches on the current device,
    so every tensor of the call must live there, and the default stream is that
    device's current stream."""
    @functools.wraps(fn)
    def call(first, *args, **kwargs):
        dev = first.device
        if dev.type != "cuda":
            raise ValueError(f"{fn.__name__}: tensors must be on a GPU, got {dev}")
        prev = getattr(_call, "device", None)
        _call.device = dev
        try:
            with torch.cuda.device(dev):
                return fn(first, *args, **kwargs)
        finally:
            _call.device = prev
    return call


def _dev(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    want = getattr(_call, "device", None)
    if want is not None and t.device != want:
        raise ValueError(f"{name} is on {t.device}; this call's tensors are on {want}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    want = getattr(_call, "device", None)
    if want is not None and s.device != want:
        raise ValueError(f"stream is on {s.device}; this call's tensors are on {want}")
    return ctypes.c_void_p(s.cuda_stream)


class PagedKVCache:
    """Caller-owned paged KV buffers plus the s3r_paged_kv struct describing them.

    k_pool [N][Hkv][P][D], v_pool [N][Hkv][D][P] (value transposed per page),
    page_table [B][max_pages] int32, seq_lens [B] int32 (device tensors).
    """

    def __init__(self, k_pool, v_pool, page_table, seq_lens, num_q_heads, total_pages_hint=0):
        if k_pool.dtype not in _KV_DTYPES:
            raise ValueError(f"kv dtype must be float32 or bfloat16, got {k_pool.dtype}")
        n_phys, hkv, P, D = k_pool.shape
        _dev(k_pool, "k_pool")
        self.device = k_pool.device
        _dev(v_pool, "v_pool", k_pool.dtype, (n_phys, hkv, D, P))
        B, maxp = page_table.shape
        _dev(page_table, "page_table", torch.int32)
        for t, name in ((v_pool, "v_pool"), (page_table, "page_table")):
            if t.device != self.device:
                raise ValueError(f"{name} is on {t.device}, k_pool on {self.device}")
        self.k_pool, self.v_pool, self.page_table = k_pool, v_pool, page_table
        self.num_q_heads = num_q_heads
        self.total_pages_hint = int(total_pages_hint)
        self.dtype = k_pool.dtype
        self.B, self.Hkv, self.P, self.D, self.max_pages = B, hkv, P, D, maxp
        self.set_seq_lens(seq_lens)

    def set_seq_lens(self, seq_lens):
        _dev(seq_lens, "seq_lens", torch.int32, (self.B,))
        if seq_lens.device != self.device:
            raise ValueError(f"seq_lens is on {seq_lens.device}, the pools on {self.device}")
        self.seq_lens = seq_lens
        self.struct = PagedKV(
            self.B, self.num_q_heads, self.Hkv, self.D, self.P, self.max_pages,
            self.total_pages_hint, _KV_DTYPES[self.dtype], self.k_pool.data_ptr(),
            self.v_pool.data_ptr(), self.page_table.data_ptr(), seq_lens.data_ptr(),
            self.k_pool.shape[0])
        return self

    def ref(self):
        return ctypes.byref(self.struct)


def version():
    return _lib.load().s3r_version()


def page_select_workspace(kv, budget_tokens):
    return _lib.load().s3r_page_select_workspace(kv.ref(), budget_tokens)


def attn_workspace(kv, n_queries, max_pages_attended):
    return _lib.load().s3r_attn_workspace(kv.ref(), n_queries, max_pages_attended)


def spec_sample_workspace(num_seqs, gamma, vocab):
    return _lib.load().s3r_spec_sample_workspace(num_seqs, gamma, vocab)


def _alloc(shape, dtype, device, stream):
    """A tensor the call allocates for itself. torch's caching allocator ties
    a block to the stream it was allocated on; when the call runs on another
    stream, the block is also recorded on that one, so it is not handed out
    again while the call's kernels may still use it."""
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        t.record_stream(stream)
    return t


def _workspace(nbytes, like, workspace, stream=None):
    if workspace is None:
        workspace = _alloc((max(int(nbytes), 1),), torch.uint8, like.device, stream)
    _dev(workspace, "workspace", torch.uint8)
    return workspace


@_on_device
def page_bounds_update(kv, bounds, first_pos=None, max_pages_touched=1, stream=None):
    """Recompute the key min/max bounds of touched pages (all pages if first_pos is None)."""
    lib = _lib.load()
    n_phys = kv.k_pool.shape[0]
    b = _dev(bounds, "bounds", kv.dtype, (n_phys, kv.Hkv, 2, kv.D))
    fp = None if first_pos is None else _dev(first_pos, "first_pos", torch.int32, (kv.B,))
    _check(lib.s3r_page_bounds_update(kv.ref(), b, fp, int(max_pages_touched), _stream(stream)),
           "s3r_page_bounds_update")
    return bounds


@_on_device
def page_select(kv, bounds, q, budget_tokens, scale, selected=None, num_selected=None,
                workspace=None, stream=None):
    """Top-k pages per (sequence, kv head) by key-bound score; returns (selected, num_selected)."""
    lib = _lib.load()
    k = budget_tokens // kv.P
    if selected is None:
        selected = _alloc((kv.B, kv.Hkv, k), torch.int32, q.device, stream)
    if num_selected is None:
        num_selected = _alloc((kv.B,), torch.int32, q.device, stream)
    ws = _workspace(page_select_workspace(kv, budget_tokens), q, workspace, stream)
    n_phys = kv.k_pool.shape[0]
    _check(lib.s3r_page_select(
        kv.ref(), _dev(bounds, "bounds", kv.dtype, (n_phys, kv.Hkv, 2, kv.D)),
        _dev(q, "q", kv.dtype, (kv.B, kv.num_q_heads, kv.D)), int(budget_tokens), float(scale),
        _dev(selected, "selected", torch.int32, (kv.B, kv.Hkv, k)),
        _dev(num_selected, "num_selected", torch.int32, (kv.B,)),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream)), "s3r_page_select")
    return selected, num_selected


_OUT_DTYPES = {torch.float32: _lib.S3R_F32, torch.bfloat16: _lib.S3R_BF16}


@_on_device
def sparse_draft_attn(kv, q, selected, scale, out=None, out_dtype=torch.float32,
                      workspace=None, stream=None):
    """One draft step's attention over the selected pages; returns out [B][Hq][D]."""
    lib = _lib.load()
    k = selected.shape[-1]
    if out is None:
        out = _alloc((kv.B, kv.num_q_heads, kv.D), out_dtype, q.device, stream)
    ws = _workspace(attn_workspace(kv, 1, k), q, workspace, stream)
    _check(lib.s3r_sparse_draft_attn(
        kv.ref(), _dev(q, "q", kv.dtype, (kv.B, kv.num_q_heads, kv.D)),
        _dev(selected, "selected", torch.int32, (kv.B, kv.Hkv, k)), k, float(scale),
        _OUT_DTYPES[out.dtype], _dev(out, "out", None, (kv.B, kv.num_q_heads, kv.D)),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream)), "s3r_sparse_draft_attn")
    return out


def sparse_draft_step_workspace(kv, budget_tokens):
    return _lib.load().s3r_sparse_draft_step_workspace(kv.ref(), budget_tokens)


@_on_device
def sparse_draft_step(kv, bounds, q, budget_tokens, scale, refresh_from=None, selected=None,
                      num_selected=None, out=None, out_dtype=torch.float32, workspace=None,
                      stream=None):
    """Bounds refresh + page select + sparse draft attention in one call;
    returns (out [B][Hq][D], selected [B][Hkv][k], num_selected [B])."""
    lib = _lib.load()
    k = budget_tokens // kv.P
    if selected is None:
        selected = _alloc((kv.B, kv.Hkv, k), torch.int32, q.device, stream)
    if num_selected is None:
        num_selected = _alloc((kv.B,), torch.int32, q.device, stream)
    if out is None:
        out = _alloc((kv.B, kv.num_q_heads, kv.D), out_dtype, q.device, stream)
    ws = _workspace(sparse_draft_step_workspace(kv, budget_tokens), q, workspace, stream)
    n_phys = kv.k_pool.shape[0]
    rf = None if refresh_from is None else _dev(refresh_from, "refresh_from", torch.int32, (kv.B,))
    _check(lib.s3r_sparse_draft_step(
        kv.ref(), _dev(bounds, "bounds", kv.dtype, (n_phys, kv.Hkv, 2, kv.D)), rf,
        _dev(q, "q", kv.dtype, (kv.B, kv.num_q_heads, kv.D)), int(budget_tokens), float(scale),
        _dev(selected, "selected", torch.int32, (kv.B, kv.Hkv, k)),
        _dev(num_selected, "num_selected", torch.int32, (kv.B,)), _OUT_DTYPES[out.dtype],
        _dev(out, "out", None, (kv.B, kv.num_q_heads, kv.D)), ctypes.c_void_p(ws.data_ptr()),
        ws.numel(), _stream(stream)), "s3r_sparse_draft_step")
    return out, selected, num_selected


@_on_device
def sparse_draft_round(kv, bounds, q, budget_tokens, gamma, scale, refresh_from=None,
                       selected=None, num_selected=None, out=None, out_dtype=torch.float32,
                       workspace=None, stream=None):
    """Draft step 0 of a round that selects once: the pages holding the round's
    gamma query positions are always kept, the rest by score; later steps pass
    the returned selection to sparse_draft_attn. Returns (out, selected,
    num_selected); the workspace is sized by sparse_draft_step_workspace."""
    lib = _lib.load()
    k = budget_tokens // kv.P
    if selected is None:
        selected = _alloc((kv.B, kv.Hkv, k), torch.int32, q.device, stream)
    if num_selected is None:
        num_selected = _alloc((kv.B,), torch.int32, q.device, stream)
    if out is None:
        out = _alloc((kv.B, kv.num_q_heads, kv.D), out_dtype, q.device, stream)
    ws = _workspace(sparse_draft_step_workspace(kv, budget_tokens), q, workspace, stream)
    n_phys = kv.k_pool.shape[0]
    rf = None if refresh_from is None else _dev(refresh_from, "refresh_from", torch.int32, (kv.B,))
    _check(lib.s3r_sparse_draft_round(
        kv.ref(), _dev(bounds, "bounds", kv.dtype, (n_phys, kv.Hkv, 2, kv.D)), rf,
        _dev(q, "q", kv.dtype, (kv.B, kv.num_q_heads, kv.D)), int(budget_tokens), int(gamma),
        float(scale), _dev(selected, "selected", torch.int32, (kv.B, kv.Hkv, k)),
        _dev(num_selected, "num_selected", torch.int32, (kv.B,)), _OUT_DTYPES[out.dtype],
        _dev(out, "out", None, (kv.B, kv.num_q_heads, kv.D)), ctypes.c_void_p(ws.data_ptr()),
        ws.numel(), _stream(stream)), "s3r_sparse_draft_round")
    return out, selected, num_selected


@_on_device
def kv_commit(kv, k_new, v_new, first_pos, bounds=None, stream=None):
    """Write k_new/v_new [B][count][Hkv][D] at positions first_pos[b] + i into the
    pools of kv and bring the touched pages' bounds up to date for kv's
    seq_lens (the committed lengths); returns bounds."""
    lib = _lib.load()
    B, count = k_new.shape[0], k_new.shape[1]
    shape = (kv.B, count, kv.Hkv, kv.D)
    n_phys = kv.k_pool.shape[0]
    b = None if bounds is None else _dev(bounds, "bounds", kv.dtype, (n_phys, kv.Hkv, 2, kv.D))
    _check(lib.s3r_kv_commit(
        kv.ref(), _dev(k_new, "k_new", kv.dtype, shape), _dev(v_new, "v_new", kv.dtype, shape),
        _dev(first_pos, "first_pos", torch.int32, (kv.B,)), int(count), b, _stream(stream)),
        "s3r_kv_commit")
    return bounds


@_on_device
def dense_verify_attn(kv, q, scale, out=None, out_dtype=torch.float32, workspace=None,
                      stream=None):
    """Causal verify attention of q [B][n_q][Hq][D] over every page; returns out like q."""
    lib = _lib.load()
    nq = q.shape[1]
    shape = (kv.B, nq, kv.num_q_heads, kv.D)
    if out is None:
        out = _alloc(shape, out_dtype, q.device, stream)
    ws = _workspace(attn_workspace(kv, nq, kv.max_pages), q, workspace, stream)
    _check(lib.s3r_dense_verify_attn(
        kv.ref(), _dev(q, "q", kv.dtype, shape), nq, float(scale), _OUT_DTYPES[out.dtype],
        _dev(out, "out", None, shape), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
        _stream(stream)), "s3r_dense_verify_attn")
    return out


@_on_device
def spec_sample(draft_logits, target_logits, draft_tokens, temperature, seed, offset,
                out_tokens=None, num_accepted=None, workspace=None, stream=None):
    """Exact speculative sampling of one round; returns (out_tokens, num_accepted)."""
    lib = _lib.load()
    B, gamma, V = draft_logits.shape
    if out_tokens is None:
        out_tokens = _alloc((B, gamma + 1), torch.int32, draft_logits.device, stream)
    if num_accepted is None:
        num_accepted = _alloc((B,), torch.int32, draft_logits.device, stream)
    ws = _workspace(spec_sample_workspace(B, gamma, V), draft_logits, workspace, stream)
    _check(lib.s3r_spec_sample(
        B, gamma, V, _dev(draft_logits, "draft_logits", torch.float32),
        _dev(target_logits, "target_logits", torch.float32, (B, gamma + 1, V)),
        _dev(draft_tokens, "draft_tokens", torch.int32, (B, gamma)), float(temperature),
        int(seed), int(offset), _dev(out_tokens, "out_tokens", torch.int32, (B, gamma + 1)),
        _dev(num_accepted, "num_accepted", torch.int32, (B,)),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream)), "s3r_spec_sample")
    return out_tokens, num_accepted


def draft_sample_workspace(num_seqs, n_rows, vocab):
    return _lib.load().s3r_draft_sample_workspace(num_seqs, n_rows, vocab)


def acceptance_rate_workspace(num_seqs, gamma, vocab):
    return _lib.load().s3r_acceptance_rate_workspace(num_seqs, gamma, vocab)


@_on_device
def draft_sample(logits, temperature, seed, offset, first_slot=0, tokens=None, workspace=None,
                 stream=None):
    """The drafter's own draws from logits [B][n_rows][V]: row r of sequence b
    samples softmax(logits[b][r] / T) with the Philox uniform U(b, first_slot + r, 2);
    returns tokens [B][n_rows] int32."""
    lib = _lib.load()
    B, R, V = logits.shape
    if tokens is None:
        tokens = _alloc((B, R), torch.int32, logits.device, stream)
    ws = _workspace(draft_sample_workspace(B, R, V), logits, workspace, stream)
    _check(lib.s3r_draft_sample(
        B, R, V, _dev(logits, "logits", torch.float32), float(temperature), int(seed), int(offset),
        int(first_slot), _dev(tokens, "tokens", torch.int32, (B, R)), ctypes.c_void_p(ws.data_ptr()),
        ws.numel(), _stream(stream)), "s3r_draft_sample")
    return tokens


@_on_device
def acceptance_rate(draft_logits, target_logits, temperature, alpha=None, workspace=None, stream=None):
    """alpha [B][gamma] float64 = sum_x min(p_i, q_i) per draft position
    (1 - alpha = TV(p_i, q_i)); target_logits holds gamma + 1 rows."""
    lib = _lib.load()
    B, gamma, V = draft_logits.shape
    if alpha is None:
        alpha = _alloc((B, gamma), torch.float64, draft_logits.device, stream)
    ws = _workspace(acceptance_rate_workspace(B, gamma, V), draft_logits, workspace, stream)
    _check(lib.s3r_acceptance_rate(
        B, gamma, V, _dev(draft_logits, "draft_logits", torch.float32),
        _dev(target_logits, "target_logits", torch.float32, (B, gamma + 1, V)), float(temperature),
        _dev(alpha, "alpha", torch.float64, (B, gamma)), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
        _stream(stream)), "s3r_acceptance_rate")
    return alpha


@_on_device
def spec_sample_noalloc(draft_logits, target_logits, draft_tokens, temperature, seed, offset,
                        out_tokens, num_accepted, stream=None):
    """spec_sample with the library's own device scratch: nothing is allocated,
    so the caller passes the outputs. Calls that may overlap on one GPU share
    that scratch and must be serialised."""
    lib = _lib.load()
    B, gamma, V = draft_logits.shape
    _check(lib.s3r_spec_sample_noalloc(
        B, gamma, V, _dev(draft_logits, "draft_logits", torch.float32),
        _dev(target_logits, "target_logits", torch.float32, (B, gamma + 1, V)),
        _dev(draft_tokens, "draft_tokens", torch.int32, (B, gamma)), float(temperature),
        int(seed), int(offset), _dev(out_tokens, "out_tokens", torch.int32, (B, gamma + 1)),
        _dev(num_accepted, "num_accepted", torch.int32, (B,)), _stream(stream)),
        "s3r_spec_sample_noalloc")
    return out_tokens, num_accepted

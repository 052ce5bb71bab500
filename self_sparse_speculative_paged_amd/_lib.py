"""ctypes view of libs3r.so (the C ABI declared in include/s3r.h).

Loading fails loudly when the library has not been built: there is no
fallback path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libs3r.so")

S3R_OK = 0
S3R_ERR_INVALID_ARGUMENT = 1
S3R_ERR_UNSUPPORTED = 2
S3R_ERR_WORKSPACE_TOO_SMALL = 3
S3R_ERR_HIP = 4
S3R_F32 = 0
S3R_BF16 = 1

EXPORTS = [
    "s3r_page_select_workspace", "s3r_attn_workspace", "s3r_spec_sample_workspace",
    "s3r_page_bounds_update", "s3r_page_select", "s3r_sparse_draft_attn",
    "s3r_dense_verify_attn", "s3r_spec_sample", "s3r_status_string", "s3r_version",
    "s3r_sparse_draft_step_workspace", "s3r_sparse_draft_step", "s3r_sparse_draft_round",
    "s3r_kv_commit", "s3r_draft_sample_workspace", "s3r_draft_sample",
    "s3r_acceptance_rate_workspace", "s3r_acceptance_rate", "s3r_spec_sample_noalloc_max_workspace",
    "s3r_spec_sample_noalloc",
]


class PagedKV(ctypes.Structure):
    """Mirror of s3r_paged_kv."""
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("total_pages_hint", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("num_phys_pages", ctypes.c_int32),
    ]


_lib = None


def load():
    """Load libs3r.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libs3r.so not found at {LIB_PATH}: build it first with "
            "`python -m self_sparse_speculative_paged_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(PagedKV)
    vp, i32, i64, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                  ctypes.c_float, ctypes.c_size_t)
    sig = {
        "s3r_page_select_workspace": (sz, [P, i32]),
        "s3r_attn_workspace": (sz, [P, i32, i32]),
        "s3r_spec_sample_workspace": (sz, [i32, i32, i32]),
        "s3r_page_bounds_update": (i32, [P, vp, vp, i32, vp]),
        "s3r_page_select": (i32, [P, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
        "s3r_sparse_draft_attn": (i32, [P, vp, vp, i32, f32, i32, vp, vp, sz, vp]),
        "s3r_dense_verify_attn": (i32, [P, vp, i32, f32, i32, vp, vp, sz, vp]),
        "s3r_sparse_draft_step_workspace": (sz, [P, i32]),
        "s3r_sparse_draft_step": (i32, [P, vp, vp, vp, i32, f32, vp, vp, i32, vp, vp, sz, vp]),
        "s3r_sparse_draft_round": (i32, [P, vp, vp, vp, i32, i32, f32, vp, vp, i32, vp, vp, sz, vp]),
        "s3r_kv_commit": (i32, [P, vp, vp, vp, i32, vp, vp]),
        "s3r_spec_sample": (i32, [i32, i32, i32, vp, vp, vp, f32, u64, u64, vp, vp, vp, sz, vp]),
        "s3r_draft_sample_workspace": (sz, [i32, i32, i32]),
        "s3r_draft_sample": (i32, [i32, i32, i32, vp, f32, u64, u64, i64, vp, vp, sz, vp]),
        "s3r_acceptance_rate_workspace": (sz, [i32, i32, i32]),
        "s3r_acceptance_rate": (i32, [i32, i32, i32, vp, vp, f32, vp, vp, sz, vp]),
        "s3r_spec_sample_noalloc_max_workspace": (sz, []),
        "s3r_spec_sample_noalloc": (i32, [i32, i32, i32, vp, vp, vp, f32, u64, u64, vp, vp, vp]),
        "s3r_status_string": (ctypes.c_char_p, [i32]),
        "s3r_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib

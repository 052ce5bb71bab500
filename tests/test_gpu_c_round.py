"""One S3R round driven from plain C (tests/c/round_gpu.c) through libs3r, with
device memory from the HIP runtime's C API and no Python or torch in the GPU
process, compared with the oracle: page bounds exactly, the page selection and
the sampled tokens within their decision windows, and the attention outputs
to the fp32 or bf16 tolerance. The C caller is built with gcc against
include/s3r.h, the in-tree libs3r.so and the HIP runtime."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle
from s3r_inputs import make_workload
from tests.oracle_io import f64, i32
from tests.parity import check_pages, check_tokens

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "self_sparse_speculative_paged_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    exe = tmp_path / "round_gpu"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c", "round_gpu.c"), "-L", LIBDIR, "-ls3r", f"-Wl,-rpath,{LIBDIR}",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-lm",
           "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def _raw(t):
    """The tensor's bytes as laid out in memory (bf16 as its 16-bit patterns)."""
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.numpy().tobytes()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_round_from_c_matches_oracle(tmp_path, kv):
    print(f"C caller round: {kv} KV", flush=True)
    exe = _build(tmp_path)
    if kv == "f32":
        cfg = "tiny_fp32"
        ctx = None
    else:
        cfg = dict(B=3, Hq=8, Hkv=2, D=128, L=None, P=16, budget=96, gamma=4, V=3000, kv_dtype="bf16",
                   draft_sd=2.0, noise_sd=0.7, temperature=1.0, heavy_pages=0)
        ctx = [700, 95, 333]
    wl = make_workload(cfg, device="cpu", seed=3, ctx=ctx)
    c = wl.cfg
    B, Hq, Hkv, D, P, gamma, V = (c[k] for k in ("B", "Hq", "Hkv", "D", "P", "gamma", "V"))
    inputs = {"k_pool": wl.k_pool, "v_pool": wl.v_pool, "page_table": wl.page_table,
              "seq_lens0": wl.seq_lens[0], "seq_lens_v": wl.seq_lens[gamma], "q_draft": wl.draft_q(0),
              "q_verify": wl.q_verify, "draft_logits": wl.draft_logits, "target_logits": wl.target_logits,
              "draft_tokens": wl.draft_tokens}
    for name, t in inputs.items():
        (tmp_path / f"{name}.bin").write_bytes(_raw(t))
    n_phys = wl.k_pool.shape[0]
    args = [str(exe), str(tmp_path), B, Hq, Hkv, D, P, wl.max_pages, n_phys, c["budget"], gamma, V,
            int(kv == "f32")]
    run = subprocess.run([str(a) for a in args], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stderr + run.stdout

    def out(name, dtype, shape):
        return np.frombuffer((tmp_path / f"{name}.bin").read_bytes(), dtype=dtype).reshape(shape)

    K, Vp, PT = f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table)
    L0, Lv = i32(wl.seq_lens[0]), i32(wl.seq_lens[gamma])
    scale = 1.0 / np.sqrt(D)
    k = c["budget"] // P

    raw = out("bounds", np.float32 if kv == "f32" else np.uint16, (n_phys, Hkv, 2, D))
    if kv == "bf16":
        raw = (raw.astype(np.uint32) << 16).view(np.float32)
    bounds = raw.astype(np.float64)
    rb = oracle.page_bounds(K, PT, L0)
    used = ~np.isnan(rb[:, 0, 0, 0])
    assert np.array_equal(bounds[used], rb[used])

    sel, nsel = out("selected", np.int32, (B, Hkv, k)), out("num_selected", np.int32, (B,))
    rsel, rn, rsc = oracle.page_select(rb, f64(wl.draft_q(0)), PT, L0, c["budget"], scale)
    check_pages(sel, nsel, rsel, rn, rsc, k)

    def close(got, ref):
        if kv == "f32":
            assert np.max(np.abs(got - ref)) / np.max(np.abs(ref)) <= 1e-5
        else:
            assert np.max(np.abs(got - ref)) <= 1e-2

    close(out("draft_out", np.float32, (B, Hq, D)).astype(np.float64),
          oracle.sparse_draft_attn(f64(wl.draft_q(0)), K, Vp, PT, L0, sel, scale))
    close(out("verify_out", np.float32, (B, gamma + 1, Hq, D)).astype(np.float64),
          oracle.dense_verify_attn(f64(wl.q_verify), K, Vp, PT, Lv, scale))

    ro, rnacc, dec = oracle.spec_sample(f64(wl.draft_logits), f64(wl.target_logits), i32(wl.draft_tokens),
                                        1.0, 0, 7)
    full = check_tokens(out("out_tokens", np.int32, (B, gamma + 1)), out("num_accepted", np.int32, (B,)),
                        ro, rnacc, dec)
    assert full >= B // 2

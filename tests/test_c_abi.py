"""include/s3r.h compiles as C99 and libs3r.so links into, and is callable from,
a plain C program (tests/c/abi_check.c). It uses only host-side queries and calls
that fail validation, so no GPU is touched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "self_sparse_speculative_paged_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_is_c99_and_library_links_from_c(tmp_path):
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"),
           "-L", LIBDIR, "-ls3r", f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stderr + run.stdout


CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
BUILD = os.path.join(ROOT, "_build")


@pytest.mark.skipif(not (os.path.exists(CLANG) and os.path.exists(HIPCC)), reason="needs the ROCm clang")
@pytest.mark.skipif(not os.path.isdir(BUILD), reason="needs the objects of a library build")
def test_host_abi_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """The C ABI layer (argument checks, plans, workspace sizes, the S3R_DEBUG
    checks' host side) rebuilt with AddressSanitizer and UBSan on the host
    pass only (the kernels' objects are the ordinary build's), driven by the
    plain C caller, also built with both sanitizers. Any report fails."""
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in ("s3r_api.cpp", "s3r_debug.cpp"):
        obj = str(tmp_path / (src + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san,
               "-I", os.path.join(ROOT, "include"), "-I", os.path.join(LIBDIR, "csrc"),
               "-c", os.path.join(LIBDIR, "csrc", src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        objs.append(obj)
    kernels = [os.path.join(BUILD, f + ".o") for f in ("s3r_attn.hip", "s3r_select.hip", "s3r_sample.hip",
                                                      "s3r_kv.hip")]
    if not all(os.path.exists(k) for k in kernels):
        pytest.skip("kernel objects missing: build the library first")
    lib = tmp_path / "libs3r_san.so"
    res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, *kernels, "-o", str(lib)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    exe = tmp_path / "abi_check_san"
    res = subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"),
                          str(lib), f"-Wl,-rpath,{tmp_path}", "-o", str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stderr[-3000:] + run.stdout

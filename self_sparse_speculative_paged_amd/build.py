"""Build libs3r.so in-tree with hipcc for gfx950.

python -m self_sparse_speculative_paged_amd.build   (or __graft_entry__.build())

The sources compile in parallel to objects under _build/ and link into
libs3r.so next to this file. hipcc's kernel resource remarks are kept in
kernel_resources.txt beside the library (registers, LDS, scratch and
occupancy per kernel); a kernel that spills to scratch is reported on stderr.
"""
import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libs3r.so")
REPORT = os.path.join(PKG, "kernel_resources.txt")
SOURCES = ["s3r_api.cpp", "s3r_debug.cpp", "s3r_attn.hip", "s3r_select.hip", "s3r_sample.hip", "s3r_kv.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU ops: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
NOISE = "is not a recognized feature for this target"


def _compile(src):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-I",
           os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    return cmd, obj, res


def _resources(text):
    """(kernel, {field: value}) from hipcc's kernel-resource-usage remarks."""
    out, cur = [], None
    for line in text.splitlines():
        m = re.search(r"remark: (Function Name|[A-Za-z ]+(?:\[[^\]]*\])?): (\S+)", line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = {}
            out.append((val, cur))
        elif cur is not None:
            cur[key] = val
    return out


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as pool:
        results = list(pool.map(_compile, srcs))
    report, spills, msgs = [], [], []
    for cmd, obj, res in results:
        text = res.stdout + res.stderr
        if res.returncode != 0:
            errs = [ln for ln in text.splitlines() if NOISE not in ln and "remark:" not in ln]
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(errs))
        msgs += [ln for ln in text.splitlines()
                 if NOISE not in ln and "remark:" not in ln and "kernel-resource-usage" not in ln]
        for name, f in _resources(text):
            report.append(f"{name} vgpr={f.get('VGPRs', '?')} agpr={f.get('AGPRs', '?')} "
                          f"sgpr={f.get('SGPRs', '?')} scratch={f.get('ScratchSize [bytes/lane]', '?')} "
                          f"lds={f.get('LDS Size [bytes/block]', '?')} "
                          f"occupancy={f.get('Occupancy [waves/SIMD]', '?')}")
            if f.get("ScratchSize [bytes/lane]", "0") not in ("0", "?"):
                spills.append(report[-1])
    tmp = LIB + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o, _ in results], "-o", tmp]
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + " ".join(link) + "\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    with open(REPORT, "w") as f:
        f.write("\n".join(sorted(report)) + "\n")
    if spills:
        print("warning: kernels spill to scratch:\n  " + "\n  ".join(spills), file=sys.stderr)
    if verbose and msgs:
        print("\n".join(msgs))
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

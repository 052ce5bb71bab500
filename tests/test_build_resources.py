"""The built kernels keep everything in registers: no kernel spills to scratch.

A spill slows a bandwidth-bound kernel by up to half (it happened once to the
page scorer and to the 64-row verify); the build records hipcc's per-kernel
resource remarks next to the library, and this test reads them.
"""
import os

import pytest

REPORT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "self_sparse_speculative_paged_amd", "kernel_resources.txt")


def test_no_kernel_spills_to_scratch():
    if not os.path.exists(REPORT):
        pytest.skip("library not built here (kernel_resources.txt is written by the build)")
    lines = [ln for ln in open(REPORT) if ln.strip()]
    assert lines, "empty resource report"
    spills = [ln.split()[0] for ln in lines if "scratch=0 " not in ln]
    assert not spills, f"kernels using scratch: {spills}"

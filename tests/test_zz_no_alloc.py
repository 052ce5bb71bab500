"""The allocation-free sampler, s3r_spec_sample_noalloc, against s3r_spec_sample
(the same kernels with a caller workspace): bit-identical tokens and accepted
counts on two calls in a row, the second with a smaller input (the scratch
keeps the first call's contents), and the size limit refused on the host.
Both also follow the oracle within the decision window."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import self_sparse_speculative_paged_amd as s3r
from self_sparse_speculative_paged_amd import _lib
from tests.parity import check_tokens


def _case(B, gamma, V, seed):
    g = torch.Generator().manual_seed(seed)
    d = torch.randn((B, gamma, V), generator=g) * 2.0
    t = torch.cat([d + torch.randn((B, gamma, V), generator=g) * 0.7,
                   torch.randn((B, 1, V), generator=g) * 2.0], dim=1)
    x = torch.from_numpy(oracle.draw_draft_tokens(d.double().numpy(), 1.0, seed=seed, offset=0))
    return d, t, x


@pytest.mark.gpu
def test_noalloc_sampler_equals_workspace_sampler():
    lib = _lib.load()
    assert lib.s3r_spec_sample_noalloc_max_workspace() == 4 << 20
    for B, gamma, V, seed in [(32, 6, 151936, 1), (5, 3, 5000, 2)]:  # the second call is smaller
        print("noalloc sampler", B, gamma, V, flush=True)
        d, t, x = _case(B, gamma, V, seed)
        dd, td, xd = d.cuda(), t.cuda(), x.int().cuda()
        ref_out, ref_n = s3r.spec_sample(dd, td, xd, 1.0, 3, 5)
        out = torch.full((B, gamma + 1), -7, dtype=torch.int32, device="cuda")
        n = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        s3r.spec_sample_noalloc(dd, td, xd, 1.0, 3, 5, out, n)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(n, ref_n), (B, gamma, V)
        ro, rn, dec = oracle.spec_sample(d.double().numpy(), t.double().numpy(), x.numpy(), 1.0, 3, 5)
        assert check_tokens(out.cpu().numpy(), n.cpu().numpy(), ro, rn, dec) >= B // 2


def test_noalloc_sampler_refuses_oversized_calls():
    """Past the scratch's 4 MiB the call returns WORKSPACE_TOO_SMALL on the host
    (the fake pointers are never touched); invalid arguments as spec_sample."""
    lib = _lib.load()
    v = ctypes.c_void_p(0x1000)
    cap = lib.s3r_spec_sample_noalloc_max_workspace()
    B = 1
    while lib.s3r_spec_sample_workspace(B, 16, 151936) <= cap:
        B *= 2
    assert lib.s3r_spec_sample_noalloc(B, 16, 151936, v, v, v, 1.0, 0, 0, v, v, None) == 3
    assert lib.s3r_spec_sample_noalloc(0, 4, 1024, v, v, v, 1.0, 0, 0, v, v, None) == 1
    assert lib.s3r_spec_sample_noalloc(2, 17, 1024, v, v, v, 1.0, 0, 0, v, v, None) == 1
    assert lib.s3r_spec_sample_noalloc(2, 4, 1024, v, v, None, 1.0, 0, 0, v, v, None) == 1
    assert np.isfinite(cap)

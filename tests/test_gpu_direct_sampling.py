"""GPU parity of direct sparse sampling: the drafter's own draws
(s3r_draft_sample) and the acceptance rate alpha = sum_x min(p, q)
(s3r_acceptance_rate), against oracle.draw_tokens and oracle.acceptance_rate
on the same seeded logits, through the C ABI.

Tolerances:
* tokens are bit-exact, except rows whose oracle draw lies within 1e-6 of a
  CDF boundary (|u * sum(q) - boundary| <= 1e-6 * sum(q)), where the kernels'
  fp32 exponentials may pick the neighbouring token; every test asserts that
  most rows are compared;
* alpha to 5e-6 absolute. A weight 2^a of the kernels carries relative error
  at most about ln(2) * 2^-23 * |a| + 2^-23 from the fp32 argument a = (x - M)
  log2(e) / T and the fp32 exp2; weights with |a| > 24 are below 2^-24 of the
  row maximum's, so every weight that matters is within about 2.1e-6
  relative. alpha <= 1 sums such weights over the normalisers, which carry
  the same bound, so |alpha_gpu - alpha| <= 2 * 2.1e-6 + fp64 rounding.
"""
import numpy as np
import pytest
import torch

import oracle
import self_sparse_speculative_paged_amd as s3r
from tests.oracle_io import i32

pytestmark = pytest.mark.gpu
DEV = "cuda"
ALPHA_TOL = 5e-6


def _logits(B, R, V, seed, sd=2.0, mask=0.0, masked_head=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((B, R, V), generator=g) * sd
    if mask > 0:
        x[torch.rand(x.shape, generator=g) < mask] = float("-inf")
        x[..., 0] = torch.randn((B, R), generator=g)  # every row keeps a finite logit
    if masked_head:
        x[..., :masked_head] = float("-inf")
    return x


def _compare_draws(got, ref, margin, min_frac=0.5):
    close = margin <= 1e-6
    assert np.array_equal(got[~close], ref[~close]), np.argwhere((got != ref) & ~close)[:5]
    assert (~close).mean() >= min_frac, (~close).mean()


@pytest.mark.parametrize("B,R,V,T,first_slot", [
    (16, 6, 151936, 1.0, 0),   # the Qwen3 vocabulary, a round's gamma = 6 rows
    (8, 3, 4099, 0.6, 2),      # a partial second chunk, T != 1, a later first slot
    (40, 1, 100, 1.0, 5),      # one position at a time, a vocabulary inside one chunk
    (4, 16, 2001, 1.0, 0),
    (6, 2, 1, 1.0, 0),         # one-token vocabulary
    (3, 2, 8191, 1.3, 7)])     # one token short of two chunks
def test_draft_sample_matches_oracle(B, R, V, T, first_slot):
    x = _logits(B, R, V, seed=V + B)
    got = s3r.draft_sample(x.to(DEV), T, seed=9, offset=4, first_slot=first_slot)
    torch.cuda.synchronize()
    ref, margin = oracle.draw_tokens(x.double().numpy(), T, 9, 4, first_slot=first_slot)
    _compare_draws(i32(got), ref, margin)
    if V == 1:
        assert np.all(i32(got) == 0)


def test_draft_sample_masked_logits():
    """Random -inf masks, a masked vocabulary tail that fills whole chunks, and
    more than 128 chunks of which the first 2 * 64 are masked in every row."""
    B, R, V, T = 4, 3, 600000, 1.0
    x = _logits(B, R, V, seed=3, mask=0.5, masked_head=2 * 64 * 4096)
    x[..., V - 3 * 4096:] = float("-inf")
    got = s3r.draft_sample(x.to(DEV), T, seed=1, offset=0)
    torch.cuda.synchronize()
    ref, margin = oracle.draw_tokens(x.double().numpy(), T, 1, 0)
    _compare_draws(i32(got), ref, margin, min_frac=0.3)
    g = i32(got)
    for b in range(B):
        for r in range(R):
            assert np.isfinite(x[b, r, g[b, r]].item()), (b, r, g[b, r])


def test_draft_sample_law_chi_square():
    """Many sequences drawing from the same row follow q (the definition), and
    one call equals one call per position with that position's first_slot."""
    from scipy import stats
    B, V, T = 4000, 64, 1.0
    row = _logits(1, 1, V, seed=5)
    x = row.expand(B, 2, V).contiguous()
    got = i32(s3r.draft_sample(x.to(DEV), T, seed=2, offset=0))
    q = oracle.softmax(row[0, 0].double().numpy(), T)
    counts = np.bincount(got[:, 0], minlength=V)
    assert stats.chisquare(counts, q * B).pvalue > 1e-3
    one = i32(s3r.draft_sample(x[:, 1:].contiguous().to(DEV), T, seed=2, offset=0, first_slot=1))
    assert np.array_equal(one[:, 0], got[:, 1])


@pytest.mark.parametrize("B,gamma,V,noise,T", [
    (16, 6, 151936, 0.5, 1.0), (8, 4, 4099, 1.35, 0.7), (32, 2, 100, 3.0, 1.0),
    (4, 16, 2001, 0.0, 1.0),   # q = p: alpha = 1
    (5, 3, 1, 1.0, 1.0)])      # one token: alpha = 1
def test_acceptance_rate_matches_oracle(B, gamma, V, noise, T):
    g = torch.Generator().manual_seed(V + gamma)
    d = torch.randn((B, gamma, V), generator=g) * 2.0
    t = torch.cat([d + torch.randn((B, gamma, V), generator=g) * noise,
                   torch.randn((B, 1, V), generator=g) * 2.0], dim=1)
    got = s3r.acceptance_rate(d.to(DEV), t.to(DEV), T).cpu().numpy()
    ref = oracle.acceptance_rate(d.double().numpy(), t.double().numpy(), T)
    assert np.max(np.abs(got - ref)) <= ALPHA_TOL, np.max(np.abs(got - ref))
    if noise == 0.0 or V == 1:
        assert np.max(np.abs(got - 1.0)) <= ALPHA_TOL


def test_acceptance_rate_masked_and_disjoint():
    """-inf masks in both rows; one position whose supports are disjoint
    (alpha = 0 exactly: every min is an exact zero); masked leading chunks of a
    vocabulary of more than 64 chunks."""
    B, gamma, V, T = 3, 4, 300000, 1.0
    g = torch.Generator().manual_seed(11)
    d = torch.randn((B, gamma, V), generator=g) * 2.0
    t = torch.cat([d + torch.randn((B, gamma, V), generator=g) * 0.7,
                   torch.randn((B, 1, V), generator=g) * 2.0], dim=1)
    d[torch.rand(d.shape, generator=g) < 0.3] = float("-inf")
    t[torch.rand(t.shape, generator=g) < 0.3] = float("-inf")
    d[..., :30 * 4096] = float("-inf")
    t[..., :30 * 4096] = float("-inf")
    d[0, 1, : V // 2] = float("-inf")
    t[0, 1, V // 2:] = float("-inf")
    got = s3r.acceptance_rate(d.to(DEV), t.to(DEV), T).cpu().numpy()
    ref = oracle.acceptance_rate(d.double().numpy(), t.double().numpy(), T)
    assert np.max(np.abs(got - ref)) <= ALPHA_TOL
    assert got[0, 1] == 0.0


def test_direct_sampling_is_deterministic():
    x = _logits(8, 4, 20000, seed=13)
    t = _logits(8, 5, 20000, seed=14)
    a1 = s3r.draft_sample(x.to(DEV), 1.0, 3, 1)
    a2 = s3r.draft_sample(x.to(DEV), 1.0, 3, 1)
    b1 = s3r.acceptance_rate(x.to(DEV), t.to(DEV), 1.0)
    b2 = s3r.acceptance_rate(x.to(DEV), t.to(DEV), 1.0)
    assert torch.equal(a1, a2) and torch.equal(b1, b2)

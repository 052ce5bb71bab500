"""Pin the oracle's Philox4x64-10 against numpy.random.Philox (an independent
implementation of the same published generator).

numpy's bit generator bumps its 256-bit counter before producing each block,
so the block numpy returns first for counter c is Philox(c + 1).
"""
import numpy as np
import pytest

import oracle

M64 = (1 << 64) - 1


def _numpy_block(counter, key):
    c = 0
    for i, w in enumerate(counter):
        c |= (int(w) & M64) << (64 * i)
    c = (c - 1) % (1 << 256)
    words = [(c >> (64 * i)) & M64 for i in range(4)]
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                          counter=np.array(words, dtype=np.uint64))
    return tuple(int(x) for x in bg.random_raw(4))


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 0, 0, 0), (0, 0)),
    ((2, 2, 3, 4), (5, 7)),
    ((M64, M64, M64, M64), (M64, M64)),
    ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
     (0x452821E638D01377, 0xBE5466CF34E90C6C)),
])
def test_philox_matches_numpy(counter, key):
    assert oracle.philox4x64_10(counter, key) == _numpy_block(counter, key)


def test_philox_random_coordinates_match_numpy():
    rng = np.random.default_rng(1234)
    for _ in range(200):
        counter = [int(x) for x in rng.integers(0, 2**63, size=4, dtype=np.int64)]
        key = [int(x) for x in rng.integers(0, 2**63, size=2, dtype=np.int64)]
        assert oracle.philox4x64_10(counter, key) == _numpy_block(counter, key)


def test_uniform_is_top53_bits_of_word0():
    for seed, off, b, slot, st in [(0, 0, 0, 0, 0), (0, 3, 17, 5, 1), (99, 1 << 40, 2, 8, 2)]:
        w0 = _numpy_block((off, b, slot, st), (seed, 0))[0]
        u = oracle.uniform(seed, off, b, slot, st)
        assert u == (w0 >> 11) / 2.0**53
        assert 0.0 <= u < 1.0


def test_uniforms_are_uniform():
    # Kolmogorov-Smirnov on 4000 coordinates: a plausible bug (wrong word, wrong
    # shift) fails this.
    from scipy import stats
    us = [oracle.uniform(7, 0, b, s, 0) for b in range(400) for s in range(10)]
    assert stats.kstest(us, "uniform").pvalue > 1e-3

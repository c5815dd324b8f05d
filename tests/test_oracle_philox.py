"""Pins of the oracle's Philox4x64-10 against numpy's independent implementation."""
import numpy as np
import pytest
from scipy import stats

from oracle.philox import MASK64, philox4x64_10, request_uniforms, uniform24


def numpy_philox_block(counter, key):
    """numpy's Philox advances its 256-bit counter before each block, so start one below."""
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    k = int(key[0]) + (int(key[1]) << 64)
    g = np.random.Philox(counter=(c - 1) % (1 << 256), key=k)
    return tuple(int(v) for v in g.random_raw(4))


def test_matches_numpy_random_cases():
    rng = np.random.default_rng(20261202)
    for _ in range(400):
        ctr = tuple(int(v) for v in rng.integers(0, 2**64, size=4, dtype=np.uint64))
        key = tuple(int(v) for v in rng.integers(0, 2**64, size=2, dtype=np.uint64))
        assert philox4x64_10(ctr, key) == numpy_philox_block(ctr, key)


@pytest.mark.parametrize("ctr,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 0, 0, 0), (0, 0)),
    ((MASK64, MASK64, MASK64, MASK64), (MASK64, MASK64)),
    ((0, 1, 2, 3), (MASK64, 0)),
    ((5, 255, 2**63, 0), (123456789, 0)),
])
def test_matches_numpy_edge_cases(ctr, key):
    assert philox4x64_10(ctr, key) == numpy_philox_block(ctr, key)


def test_request_uniforms_use_words_0_and_1():
    seed, b, i, off = 0xDEADBEEF12345678, 17, 3, 99
    w = numpy_philox_block((i, b, off, 0), (seed, 0))
    assert request_uniforms(seed, b, i, off) == ((w[0] >> 40) / 2**24, (w[1] >> 40) / 2**24)


def test_uniform24_grid_and_range():
    assert uniform24(0) == 0.0
    assert uniform24(MASK64) == 1.0 - 2.0**-24
    assert uniform24(1 << 40) == 2.0**-24
    assert uniform24((1 << 40) - 1) == 0.0
    # exactly representable in fp32
    u = uniform24(0x9E3779B97F4A7C15)
    assert float(np.float32(u)) == u


def test_uniforms_are_uniform_and_distinct_per_key():
    us = []
    for seed in range(200):
        for b in range(5):
            for i in range(6):
                ua, us_ = request_uniforms(seed, b, i, 7)
                us.extend((ua, us_))
    us = np.asarray(us)
    assert stats.kstest(us, "uniform").pvalue > 1e-4
    assert len(np.unique(us)) > 0.999 * len(us)
    # different position, request, offset and seed each change the draw
    base = request_uniforms(1, 2, 3, 4)
    for args in [(1, 2, 4, 4), (1, 3, 3, 4), (1, 2, 3, 5), (2, 2, 3, 4)]:
        assert request_uniforms(*args) != base

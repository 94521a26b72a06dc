"""Pins for the oracle's generator: Philox4x64-10 and the 53-bit uniforms.

numpy.random.Philox is an independent implementation of Philox4x64-10
(Salmon et al., SC'11); it increments its 256-bit counter before producing a
block, so its first block from counter c is Philox(c + 1).
"""
import numpy as np
import pytest
from scipy import stats

MASK64 = (1 << 64) - 1


def numpy_block(counter, key):
    """Philox4x64-10(counter, key) computed by numpy (counter given as 4 words)."""
    c = counter[0] | (counter[1] << 64) | (counter[2] << 128) | (counter[3] << 192)
    c = (c - 1) % (1 << 256)
    words = [(c >> (64 * j)) & MASK64 for j in range(4)]
    bg = np.random.Philox(counter=np.array(words, dtype=np.uint64),
                          key=np.array(key, dtype=np.uint64))
    return [int(v) for v in bg.random_raw(4)]


def test_philox_matches_numpy_random_vectors(ora):
    rng = np.random.default_rng(12345)
    for _ in range(200):
        ctr = [int(v) for v in rng.integers(0, 2**63, size=4, dtype=np.int64)]
        ctr = [c ^ (int(rng.integers(0, 2)) << 63) for c in ctr]
        key = [int(v) for v in rng.integers(0, 2**63, size=2, dtype=np.int64)]
        got = [int(v) for v in ora.philox4x64_10(ctr, key)]
        assert got == numpy_block(ctr, key)


def test_philox_edge_counters(ora):
    for ctr, key in [([0, 0, 0, 0], [0, 0]),
                     ([MASK64, MASK64, MASK64, MASK64], [MASK64, MASK64]),
                     ([1, 0, 0, 0], [0, 0]),
                     ([0, 1, 0, 0], [7, 0]),
                     ([3, 5, 0, 0], [0, 11])]:
        got = [int(v) for v in ora.philox4x64_10(ctr, key)]
        assert got == numpy_block(ctr, key)


def test_uniform_uses_word0_for_acceptance_and_word1_for_additional(ora):
    rng = np.random.default_rng(7)
    for _ in range(100):
        seed = int(rng.integers(0, 2**63))
        skey = int(rng.integers(0, 2**63))
        rnd = int(rng.integers(1, 2**31))
        i = int(rng.integers(1, 66))
        w = numpy_block([rnd, i, 0, 0], [seed, skey])
        u0 = ora.uniform(seed, skey, rnd, i, 0)
        u1 = ora.uniform(seed, skey, rnd, i, 1)
        assert u0 == (w[0] >> 11) / 2.0**53
        assert u1 == (w[1] >> 11) / 2.0**53
        for u in (u0, u1):
            assert 0.0 <= u < 1.0
            assert float(u * 2.0**53).is_integer()


def test_uniforms_are_uniform(ora):
    n = 200_000
    us = np.array([ora.uniform(0, s % 97, 1 + s // 97, 1 + s % 13, s & 1) for s in range(n)])
    assert stats.kstest(us, "uniform").pvalue > 1e-3


def test_distinct_positions_purposes_sessions_give_distinct_uniforms(ora):
    seen = set()
    for skey in range(4):
        for rnd in (1, 2):
            for i in range(1, 66):
                for purpose in (0, 1):
                    seen.add(ora.uniform(0, skey, rnd, i, purpose))
    assert len(seen) == 4 * 2 * 65 * 2

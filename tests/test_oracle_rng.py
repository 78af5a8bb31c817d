"""Pins of the oracle's counter-based generator (Philox4x64-10, Salmon et al., SC 2011), which
supplies the sampling verifier's uniforms (DScale Sec. III-D, Prefix verifier, sampling mode).

The raw 64-bit words are compared with numpy's independent Philox4x64-10 bit generator
(numpy advances its 256-bit counter before each block, so numpy's counter c yields the
oracle's blocks c + 1, c + 2, ...), across keys, counters with a carry into the second
word and lengths that end inside a block.  The uniforms are checked for their lattice
(multiples of 2^-24 in [0, 1)), their distribution (Kolmogorov-Smirnov) and the
independence of streams under different keys and counters."""
import numpy as np
import pytest
from scipy import stats

import oracle


@pytest.mark.parametrize("key,counter", [(0, 0), (7 + (9 << 64), 5), (2**128 - 1, 123456789),
                                         (0xDEADBEEF, 2**64 - 3), (1 << 100, (1 << 64) + 17)])
def test_raw_words_equal_numpy_philox(key, counter):
    n = 4 * 37
    k = np.array([key & (2**64 - 1), key >> 64], np.uint64)
    c = np.array([counter & (2**64 - 1), counter >> 64, 0, 0], np.uint64)
    ref = np.random.Philox(counter=c, key=k).random_raw(n)
    got = oracle.philox_raw(key, counter + 1, n)
    assert np.array_equal(got, ref)


def test_partial_block_is_a_prefix():
    full = oracle.philox_raw(42, 1000, 16)
    for n in (0, 1, 2, 3, 5, 15):
        assert np.array_equal(oracle.philox_raw(42, 1000, n), full[:n])
    # a stream started one block later is the same stream shifted by four words
    assert np.array_equal(oracle.philox_raw(42, 1001, 12), full[4:])


def test_counter_wraps_modulo_2_128():
    # the block after counter 2^128 - 1 is the block at counter 0 (no carry into the high words)
    key = 0x5A5A << 70
    assert np.array_equal(oracle.philox_raw(key, 2**128 - 1, 8)[4:], oracle.philox_raw(key, 0, 4))
    # the carry out of the low word reaches the high word: counter 2^64 - 1, then 2^64
    assert np.array_equal(oracle.philox_raw(key, 2**64 - 1, 8)[4:], oracle.philox_raw(key, 2**64, 4))


def test_uniforms_lattice_and_distribution():
    u = oracle.philox_uniforms(2024, 0, 1 << 20).astype(np.float64)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert np.all(u * 2**24 == np.floor(u * 2**24))
    raw = oracle.philox_raw(2024, 0, 1 << 20)
    assert np.array_equal(u * 2**24, (raw >> np.uint64(40)).astype(np.float64))
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / u.size)


def test_streams_are_independent():
    a = oracle.philox_uniforms(1, 0, 1 << 16).astype(np.float64)
    b = oracle.philox_uniforms(2, 0, 1 << 16).astype(np.float64)
    c = oracle.philox_uniforms(1, 1 << 20, 1 << 16).astype(np.float64)
    for x, y in ((a, b), (a, c), (b, c)):
        assert abs(np.corrcoef(x, y)[0, 1]) < 5 / np.sqrt(x.size)
    # neighbouring words of one block are uncorrelated too
    assert abs(np.corrcoef(a[0::4], a[1::4])[0, 1]) < 5 / np.sqrt(a.size / 4)


def test_errors():
    with pytest.raises(oracle.OracleError):
        oracle.philox_raw(-1, 0, 4)
    with pytest.raises(oracle.OracleError):
        oracle.philox_uniforms(0, 2**128, 4)

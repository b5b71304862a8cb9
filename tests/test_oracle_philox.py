"""Pins of the oracle's generator: Philox4x32-10, the word stream, the
word-to-float map and randint.

Page "(11) FusedNormalization", section 10: every random number is fixed by
(seed, offset) through a Philox counter-based generator.  The generator's
own definition is Salmon et al., SC'11; its published known-answer vectors
and PyTorch's independent header implementation pin it here.
"""
from __future__ import annotations

import numpy as np
import pytest

from conftest import read_golden


def test_philox_known_answer_vectors(orc):
    rows = read_golden("philox4x32_10_kat.txt")
    assert len(rows) == 3
    for row in rows:
        v = [int(x, 16) for x in row]
        ctr, key, expect = v[0:4], v[4:6], v[6:10]
        got = orc.philox4x32_10(ctr, key)
        assert [int(x) for x in got] == expect, row


def test_word_stream_matches_torch_philox(orc, torch_philox):
    """Word k of sample n = output k%4 of block k/4 with counter (block, n)
    and key seed: the same layout as at::Philox4_32(seed, subsequence=n,
    offset=block)."""
    rng = np.random.default_rng(7)
    cases = [(0, 0), (123, 0), (123, 255), (2**64 - 1, 2**40 + 3), (0xDEADBEEFCAFEF00D, 2**32 - 1)]
    cases += [(int(rng.integers(0, 2**63)), int(rng.integers(0, 2**40))) for _ in range(20)]
    for seed, n in cases:
        ref = torch_philox(seed, n, 0, 24)
        got = np.array([orc.word(seed, n, k) for k in range(24)], np.uint32)
        np.testing.assert_array_equal(got, ref, err_msg=f"seed={seed} n={n}")
    # a block offset far from zero, with a carry into the high counter word
    seed, n, block = 99, 5, 2**32 - 1
    ref = torch_philox(seed, n, block, 8)
    got = np.array([orc.word(seed, n, 4 * block + k) for k in range(8)], np.uint32)
    np.testing.assert_array_equal(got, ref)


def test_streams_differ_by_seed_and_sample(orc):
    a = orc.words(123, 0)
    assert not np.array_equal(a, orc.words(124, 0))
    assert not np.array_equal(a, orc.words(123, 1))
    np.testing.assert_array_equal(a, orc.words(123, 0))  # stateless


def test_u01_closed_forms(orc):
    assert orc.u01(0) == 0.0
    assert orc.u01(0xFF) == 0.0  # the low 8 bits are dropped
    assert orc.u01(0x100) == 2.0**-24
    assert orc.u01(0x80000000) == 0.5
    assert orc.u01(0x7FFFFFFF) == 0.5 - 2.0**-24
    assert orc.u01(0xFFFFFFFF) == 1.0 - 2.0**-24
    ws = np.random.default_rng(1).integers(0, 2**32, 2000, dtype=np.uint64)
    for w in ws:
        assert orc.u01(int(w)) == (int(w) >> 8) / 2.0**24


@pytest.mark.parametrize("lo,hi", [(0, 0), (0, 1), (0, 2), (0, 223), (3, 17), (0, 2**24)])
def test_randint_inclusive_and_exact(orc, lo, hi):
    span = hi - lo + 1
    assert orc.randint(lo, hi, 0) == lo
    assert orc.randint(lo, hi, 0xFFFFFFFF) == hi
    # value r is returned exactly for w in [ceil((r-lo) 2^32 / span), ceil((r-lo+1) 2^32 / span))
    for r in sorted({lo, hi, lo + span // 2, lo + span // 3}):
        first = -((-(r - lo) * 2**32) // span)
        assert orc.randint(lo, hi, first) == r
        if first > 0:
            assert orc.randint(lo, hi, first - 1) == r - 1

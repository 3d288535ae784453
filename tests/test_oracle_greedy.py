"""Pins of oracle.ref.greedy_token (the index the fused GEMV + greedy
selection must produce): hand cases for ties, signed zeros, negatives and
NaN, and agreement with numpy's first-occurrence argmax (which also returns
the first NaN) on random fp16 vectors, with and without NaN entries."""

import numpy as np
import pytest

from oracle import ref


def test_hand_cases():
    assert ref.greedy_token([1.0]) == 0
    assert ref.greedy_token([0.5, 2.0, 2.0, -3.0]) == 1          # first of a tie
    assert ref.greedy_token([-5.0, -1.0, -2.0]) == 1             # all negative
    assert ref.greedy_token(np.array([-0.0, 0.0], np.float16)) == 0   # -0 == +0
    assert ref.greedy_token(np.array([0.0, -0.0, 0.0], np.float16)) == 0
    assert ref.greedy_token(np.array([-np.inf, 7], np.float16)) == 1
    assert ref.greedy_token(np.array([3, -2, 3], np.int32)) == 0
    with pytest.raises(ValueError):
        ref.greedy_token([])


def test_matches_first_argmax():
    rng = np.random.default_rng(5)
    for n in (2, 17, 1000):
        y = (rng.standard_normal(n) * 4).astype(np.float16)    # many ties in fp16
        assert ref.greedy_token(y) == int(np.argmax(y))


def test_nan_rule():
    nan = np.float16(np.nan)
    assert ref.greedy_token(np.array([1, nan, 2], np.float16)) == 1          # NaN above a number
    assert ref.greedy_token(np.array([np.inf, nan], np.float16)) == 1        # and above +inf
    assert ref.greedy_token(np.array([nan, np.inf, nan], np.float16)) == 0   # first NaN
    neg_nan = np.array([0xFE00], np.uint16).view(np.float16)[0]             # sign bit set
    assert ref.greedy_token(np.array([5, neg_nan, nan], np.float16)) == 1    # either sign
    assert ref.greedy_token(np.array([-np.inf, -np.inf], np.float16)) == 0


def test_nan_matches_numpy_argmax():
    rng = np.random.default_rng(6)
    for n in (2, 33, 500):
        y = (rng.standard_normal(n) * 4).astype(np.float16)
        y[rng.integers(0, n, 1 + n // 50)] = np.nan
        assert ref.greedy_token(y) == int(np.argmax(y))

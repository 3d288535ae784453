"""Pins of oracle.ref.greedy_token (the index the fused GEMV + greedy
selection must produce): hand cases for ties, signed zeros and negatives,
and agreement with numpy's first-occurrence argmax on random fp16 vectors."""

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

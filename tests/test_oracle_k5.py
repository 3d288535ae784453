"""Pins of the K5 code space (TKintegers K5, "What is K5?": five balanced
trits, 243 values, one byte per code): exhaustive over every code."""

import os

import numpy as np

from oracle import quant, ref

GOLD = os.path.join(os.path.dirname(__file__), "golden", "k5_code_space.txt")


def _gold():
    out = {}
    for line in open(GOLD):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            out[k] = int(v)
    return out


def test_code_space_exhaustive():
    g = _gold()
    codes = np.arange(3 ** g["trits"])
    assert codes.size == g["values"]
    assert codes.max() < 256 ** g["bytes_per_code"]
    trits = ref.k5_trits(codes)
    assert trits.shape == (243, 5)
    assert set(np.unique(trits).tolist()) == {-1, 0, 1}
    vals = ref.k5_value(codes)
    # image is exactly the integers -121..121, bijectively
    assert vals.min() == -121 and vals.max() == 121
    assert np.array_equal(np.sort(vals), np.arange(-121, 122))
    # sum of 3^i for i < 5 is 121, so value(c) = c - 121
    assert sum(3 ** i for i in range(5)) == 121
    assert np.array_equal(vals, codes - 121)
    # every trit pattern appears exactly once
    assert len({tuple(t) for t in trits.tolist()}) == 243


def test_trit_examples():
    # c = 0: all digits 0 -> all trits -1 -> -121 ; c = 242: all digits 2 -> +121
    assert ref.k5_trits(0).tolist() == [-1] * 5
    assert ref.k5_trits(242).tolist() == [1] * 5
    # c = 121 is the zero code: digits 1,1,1,1,1
    assert ref.k5_trits(121).tolist() == [0] * 5
    # c = 1 -> digits (1,0,0,0,0) -> trits (0,-1,-1,-1,-1) -> -120
    assert ref.k5_value(1) == -120


def test_quantizer_lossless_on_grid():
    # scale 2^-7 exactly: a = 121 * 2^-7, so a/121 = 2^-7 (exact in fp32, fp16)
    v = np.concatenate([np.arange(-121, 122), np.arange(-121, -108)])
    assert v.size == 256
    W = (v.astype(np.float32) * np.float32(2.0 ** -7)).reshape(2, 128)
    c, s = quant.quantize_k5(W)
    assert np.all(s == np.float16(2.0 ** -7))
    assert np.array_equal(c.astype(np.int64).ravel(), v + 121)
    w_deq = ref.dequant_k5(c, s)
    assert np.array_equal(w_deq.astype(np.float32), W)


def test_quantizer_rounding_half_even():
    # scale 1/128 again (group absmax 121/128); values at +-0.5 and +-1.5 steps
    base = np.zeros(128, np.float32)
    base[0] = np.float32(121 / 128)
    base[1] = np.float32(0.5 / 128)    # rint(0.5) = 0
    base[2] = np.float32(1.5 / 128)    # rint(1.5) = 2
    base[3] = np.float32(-2.5 / 128)   # rint(-2.5) = -2
    c, s = quant.quantize_k5(base[None, :])
    assert s[0, 0] == np.float16(1 / 128)
    assert (c[0, :4].astype(int) - 121).tolist() == [121, 0, 2, -2]


def test_degenerate_group():
    c, s = quant.quantize_k5(np.zeros((1, 128), np.float32))
    assert s[0, 0] == 1.0 and np.all(c == 121)
    assert np.all(ref.dequant_k5(c, s) == 0)

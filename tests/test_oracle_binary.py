"""Pins of the binary path: the XOR-popcount identity (Whetstone, "Measured
hardware facts") by brute force over every pair of {-1,+1} vectors with
K <= 10, plus parity, range and closed-form special cases."""

import numpy as np
import pytest

from oracle import pack, quant, ref


def _all_vectors(K):
    idx = np.arange(1 << K, dtype=np.int64)
    bits = ((idx[:, None] >> np.arange(K)) & 1).astype(np.uint8)  # bit=1 -> -1
    vals = (1 - 2 * bits.astype(np.int64))
    return bits, vals


@pytest.mark.parametrize("K", list(range(1, 11)))
def test_identity_brute_force(K):
    bits, vals = _all_vectors(K)
    # pad to 32 columns: padding bits are 0 in both operands and cancel in XOR
    padded = np.zeros((bits.shape[0], 32), dtype=np.uint8)
    padded[:, :K] = bits
    words = pack.pack_bits(padded)[:, 0]
    dots = vals @ vals.T  # every pair
    for i in range(bits.shape[0]):
        y = ref.bin_gemv(words[:, None], words[i:i + 1], K)
        assert np.array_equal(y.astype(np.int64), dots[:, i])


def test_sign_bits_polarity():
    # {-1,+1} packed as bits {1,0}
    w = np.array([[-1, 1, -1, -1] * 8], dtype=np.float32)
    b = quant.sign_bits(w)
    assert b[0, :4].tolist() == [1, 0, 1, 1]
    assert quant.sign_bits(np.array([[-0.0, 0.0]], np.float32)).tolist() == [[0, 0]]


def test_random_vs_int_dot_and_invariants():
    rng = np.random.default_rng(123)
    for K in (32, 96, 896):
        W = (1 - 2 * rng.integers(0, 2, (17, K))).astype(np.float32)
        x = (1 - 2 * rng.integers(0, 2, K)).astype(np.float32)
        wb = pack.pack_bits(quant.sign_bits(W))
        xb = pack.pack_bits(quant.sign_bits(x[None, :]))[0]
        y = ref.bin_gemv(wb, xb, K).astype(np.int64)
        assert np.array_equal(y, ref.bin_dot(W, x))
        assert np.all((y - K) % 2 == 0)        # y = K (mod 2)
        assert np.all(np.abs(y) <= K)


def test_all_plus_x_counts_negatives():
    rng = np.random.default_rng(5)
    K = 128
    W = (1 - 2 * rng.integers(0, 2, (9, K))).astype(np.float32)
    wb = pack.pack_bits(quant.sign_bits(W))
    xb = np.zeros(K // 32, dtype=np.uint32)    # all +1
    y = ref.bin_gemv(wb, xb, K).astype(np.int64)
    assert np.array_equal(y, K - 2 * (W < 0).sum(axis=1))


def test_global_flip_invariance():
    rng = np.random.default_rng(6)
    K = 64
    wb = rng.integers(0, 2**32, (4, K // 32), dtype=np.uint64).astype(np.uint32)
    xb = rng.integers(0, 2**32, K // 32, dtype=np.uint64).astype(np.uint32)
    a = ref.bin_gemv(wb, xb, K)
    b = ref.bin_gemv(~wb, ~xb, K)
    assert np.array_equal(a, b)

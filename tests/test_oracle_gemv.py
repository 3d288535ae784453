"""Pins of the fp64 GEMV / GEMM definitions and the tolerance bound: brute force
with exactly-rounded sums on tiny non-square inputs (a transposed operand
fails), closed forms and special cases."""

import math

import numpy as np

from oracle import pack, quant, ref


def test_gemv_brute_force_tiny():
    rng = np.random.default_rng(3)
    W = rng.standard_normal((5, 7))
    x = rng.standard_normal(7)
    y = ref.gemv(W, x)
    for n in range(5):
        exact = math.fsum(W[n, k] * x[k] for k in range(7))
        assert abs(y[n] - exact) <= 1e-12 * (1 + abs(exact))
    assert y.shape == (5,)


def test_gemm_brute_force_tiny():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((3, 6))
    W = rng.standard_normal((4, 6))
    Y = ref.gemm(X, W)
    assert Y.shape == (3, 4)
    for m in range(3):
        for n in range(4):
            exact = math.fsum(X[m, k] * W[n, k] for k in range(6))
            assert abs(Y[m, n] - exact) <= 1e-12 * (1 + abs(exact))
        assert np.allclose(Y[m], ref.gemv(W, X[m]), rtol=0, atol=1e-12)


def test_bound_closed_form():
    W = np.array([[1.0, -2.0], [0.0, 0.0]])
    x = np.array([3.0, 4.0])
    assert np.allclose(ref.gemv_bound(W, x), [2e-3 * 11.0, 0.0])
    ok, worst = ref.check_within([-5.0 + 0.02, 0.0], ref.gemv(W, x), ref.gemv_bound(W, x))
    assert ok and worst < 1
    ok, _ = ref.check_within([-5.0 + 0.03, 0.0], ref.gemv(W, x), ref.gemv_bound(W, x))
    assert not ok
    # a zero bound requires an exact result
    ok, worst = ref.check_within([-5.0, 1e-30], ref.gemv(W, x), ref.gemv_bound(W, x))
    assert not ok and worst == np.inf


def _packed_int4(W):
    q, s, z = quant.quantize_int4_g128(W)
    return pack.pack_int4(q), pack.pack_int4_meta(s, z)


def test_gemv_unit_vector_selects_column():
    rng = np.random.default_rng(9)
    W = rng.standard_normal((6, 256), dtype=np.float32) * np.float32(0.02)
    codes, meta = _packed_int4(W)
    w_deq = ref.dequant_int4(codes, meta, 256)
    for k in (0, 5, 127, 128, 255):
        e = np.zeros(256, np.float16)
        e[k] = 1
        assert np.array_equal(ref.gemv(w_deq, e), w_deq[:, k])


def test_gemv_zero_cases():
    rng = np.random.default_rng(10)
    W = rng.standard_normal((4, 128), dtype=np.float32)
    codes, meta = _packed_int4(W)
    w_deq = ref.dequant_int4(codes, meta, 128)
    assert np.all(ref.gemv(w_deq, np.zeros(128)) == 0)
    # all codes equal to the zero point -> the row is exactly zero
    codes0, meta0 = _packed_int4(np.zeros((3, 256), np.float32))
    assert np.all(ref.gemv(ref.dequant_int4(codes0, meta0, 256), rng.standard_normal(256)) == 0)


def test_gemv_constant_rows_closed_form():
    # grid-aligned rows: hi - lo = 15 * 2^-k so the scale is exact and the
    # quantizer is lossless (0.9375 = 15/16 -> s = 1/16, q = 15, z = 0;
    # -15/32 -> s = 1/32, z = 15, q = 0); x = ones -> y = row sum.
    W = np.zeros((2, 128), np.float32)
    W[0, :64] = 0.9375
    W[1, ::2] = -15 / 32
    codes, meta = _packed_int4(W)
    w_deq = ref.dequant_int4(codes, meta, 128)
    assert np.array_equal(w_deq.astype(np.float32), W)
    y = ref.gemv(w_deq, np.ones(128, np.float16))
    assert y.tolist() == [60.0, -30.0]


def test_dequant_tern_and_k5_agree_with_definition():
    rng = np.random.default_rng(12)
    W = rng.standard_normal((3, 256), dtype=np.float32) * np.float32(0.02)
    c, s = quant.quantize_k5(W)
    d = ref.dequant_k5(c, s)
    expect = np.repeat(s.astype(np.float64), 128, 1) * (c.astype(np.float64) - 121)
    assert np.array_equal(d, expect)
    t, st = quant.quantize_tern_g128(W)
    dt = ref.dequant_tern(pack.pack_tern(t), st, 256)
    assert set(np.unique(np.sign(dt)).tolist()) <= {-1.0, 0.0, 1.0}

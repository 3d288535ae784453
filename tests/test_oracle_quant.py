"""Pins of the int4-g128 and ternary quantizers: hand-worked groups whose
arithmetic is exact (grid-aligned weights), rounding ties, degenerate groups,
error bounds, and the sequential absmean against a scalar loop."""

import numpy as np
import pytest

from oracle import pack, quant, ref


def _int4_roundtrip(W):
    q, s, z = quant.quantize_int4_g128(W)
    codes = pack.pack_int4(q)
    meta = pack.pack_int4_meta(s, z)
    return q, s, z, ref.dequant_int4(codes, meta, W.shape[1])


def test_int4_lossless_on_grid():
    # Weights on the 1/16 grid spanning [-0.5, 0.4375]: hi - lo = 15/16, so
    # s = 1/16 exactly, z = rint(0.5 * 16) = 8 and q = 16 w + 8.
    k = np.tile(np.arange(16), 8)
    W = ((k.astype(np.float32) - 8) / np.float32(16))[None, :]
    q, s, z, w_deq = _int4_roundtrip(W)
    assert s[0, 0] == np.float16(1 / 16) and z[0, 0] == 8
    assert np.array_equal(q[0].astype(int), k)
    assert np.array_equal(w_deq.astype(np.float32), W)


def test_int4_rounding_half_even():
    # same group range (s = 1/16, z = 8) plus values at half steps
    W = np.zeros((1, 128), np.float32)
    W[0, 0], W[0, 1] = -0.5, 0.4375
    W[0, 2] = 0.5 / 16     # w/s = 0.5  -> 0  -> q = 8
    W[0, 3] = 1.5 / 16     # 1.5 -> 2  -> q = 10
    W[0, 4] = -2.5 / 16    # -2.5 -> -2 -> q = 6
    W[0, 5] = 3.5 / 16     # 3.5 -> 4  -> q = 12
    q, s, z, _ = _int4_roundtrip(W)
    assert q[0, :6].tolist() == [0, 15, 8, 10, 6, 12]


def test_int4_positive_group_has_zero_point_zero():
    # all weights >= 0: the range is widened to include 0, so lo = 0, z = 0,
    # and the largest weight gets code 15.
    W = np.linspace(0.1, 0.5, 128, dtype=np.float32)[None, :]
    q, s, z, w_deq = _int4_roundtrip(W)
    assert z[0, 0] == 0
    assert q[0, -1] == 15
    assert s[0, 0] == np.float16(np.float32(0.5) / np.float32(15))


def test_int4_negative_constant_group():
    W = np.full((1, 128), -0.3, np.float32)
    q, s, z, w_deq = _int4_roundtrip(W)
    s16 = np.float16(np.float32(0.3) / np.float32(15))
    assert s[0, 0] == s16
    assert z[0, 0] == 15 and np.all(q == 0)
    assert np.allclose(w_deq, -15 * float(s16))


@pytest.mark.parametrize("val", [0.0, 1e-9, -1e-9])
def test_int4_degenerate_groups(val):
    W = np.full((2, 256), val, np.float32)
    q, s, z, w_deq = _int4_roundtrip(W)
    # scale underflows fp16 -> guarded to 1.0; every code is the zero point 0
    assert np.all(s == 1.0) and np.all(z == 0) and np.all(q == 0)
    assert np.all(w_deq == 0)
    assert not np.any(np.isnan(w_deq))


def test_int4_error_bound_random():
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((64, 512), dtype=np.float32) * np.float32(0.02))
    q, s, z, w_deq = _int4_roundtrip(W)
    assert q.max() <= 15
    assert np.all(z.astype(np.float32) == np.rint(z.astype(np.float32)))
    G = W.reshape(64, 4, 128).astype(np.float64)
    D = w_deq.reshape(64, 4, 128)
    lo = np.minimum(G.min(2), 0)
    hi = np.maximum(G.max(2), 0)
    sf = s.astype(np.float64)
    slack = sf / 2 + np.abs(hi - lo - 15 * sf) + 1e-12
    assert np.all(np.abs(G - D) <= slack[:, :, None])


def test_tern_on_grid():
    # half the weights +-0.5, half 0: sum |w| = 32, mean = 0.25 = s;
    # w/s = +-2 clips to +-1; 0 stays 0.
    W = np.zeros((1, 128), np.float32)
    W[0, :32] = 0.5
    W[0, 32:64] = -0.5
    q, s = quant.quantize_tern_g128(W)
    assert s[0, 0] == np.float16(0.25)
    assert q[0, :32].tolist() == [2] * 32
    assert q[0, 32:64].tolist() == [0] * 32
    assert q[0, 64:].tolist() == [1] * 64
    w_deq = ref.dequant_tern(pack.pack_tern(q), s, 128)
    assert np.all(w_deq[0, :32] == 0.25) and np.all(w_deq[0, 32:64] == -0.25)


def test_tern_small_values_round_to_zero():
    W = np.full((1, 128), 0.1, np.float32)
    W[0, 0] = 0.02      # mean ~0.0994: 0.02/0.0994 = 0.2 -> 0 ; 0.1 -> 1
    q, s = quant.quantize_tern_g128(W)
    assert q[0, 0] == 1 and np.all(q[0, 1:] == 2)


def test_tern_absmean_is_sequential_sum():
    rng = np.random.default_rng(11)
    G = rng.standard_normal((5, 128), dtype=np.float32) * np.float32(0.02)
    got = quant.absmean_sequential(G)
    for r in range(5):
        acc = np.float32(0)
        for v in G[r]:
            acc = np.float32(acc + np.float32(abs(v)))
        assert got[r] == np.float32(acc / np.float32(128))


def test_tern_degenerate():
    q, s = quant.quantize_tern_g128(np.zeros((1, 128), np.float32))
    assert s[0, 0] == 1.0 and np.all(q == 1)


def test_relative_error_sanity():
    # Statistical sanity, not a pin: the page's weight relative errors are on
    # trained weights (int4 g128 ~0.11, ternary ~0.54); Gaussian weights give
    # values of the same size.
    rng = np.random.default_rng(1)
    W = rng.standard_normal((256, 896), dtype=np.float32) * np.float32(0.02)
    _, _, _, d4 = _int4_roundtrip(W)
    qt, st = quant.quantize_tern_g128(W)
    dt = ref.dequant_tern(pack.pack_tern(qt), st, 896)
    ck, sk = quant.quantize_k5(W)
    dk = ref.dequant_k5(ck, sk)
    rel = lambda D: np.linalg.norm(W - D) / np.linalg.norm(W)  # noqa: E731
    assert 0.08 < rel(d4) < 0.12
    assert 0.45 < rel(dt) < 0.56
    assert rel(dk) < 0.01


# ---- int2 g128 (Whetstone, "int2 g128": 2-bit codes, int4-style metadata) ----

def _int2_roundtrip(W):
    q, s, z = quant.quantize_int2_g128(W)
    return q, s, z, ref.dequant_int2(pack.pack_int2(q), pack.pack_int4_meta(s, z), W.shape[1])


def test_int2_lossless_on_grid():
    # weights on the 1/4 grid spanning [-0.5, 0.25]: hi - lo = 3/4, s = 1/4
    # exactly, z = 2 and q = 4 w + 2
    k = np.tile(np.arange(4), 32)
    W = ((k.astype(np.float32) - 2) / np.float32(4))[None, :]
    q, s, z, w = _int2_roundtrip(W)
    assert s[0, 0] == np.float16(0.25) and z[0, 0] == 2
    assert np.array_equal(q[0].astype(int), k)
    assert np.array_equal(w.astype(np.float32), W)


def test_int2_rounding_half_even():
    W = np.zeros((1, 128), np.float32)
    W[0, 0], W[0, 1] = -0.5, 0.25          # s = 0.25, z = 2
    W[0, 2] = 0.125                        # w/s = 0.5 -> 0 (half even) -> q = 2
    W[0, 3] = -0.375                       # -1.5 -> -2 -> q = 0
    W[0, 4] = -0.125                       # -0.5 -> -0 -> q = 2
    q, s, z, w = _int2_roundtrip(W)
    assert q[0, :5].tolist() == [0, 3, 2, 0, 2]


def test_int2_codes_are_nearest_level():
    """Brute force: each code is the nearest of the four levels s*(q - z)
    (ties excluded), and the dequantized weight is within half a step of every
    weight inside the group's range."""
    rng = np.random.default_rng(21)
    W = (rng.standard_normal((5, 256)) * 0.02).astype(np.float32)
    q, s, z, w = _int2_roundtrip(W)
    for n in range(5):
        for g in range(2):
            sf, zf = float(s[n, g]), float(z[n, g])
            levels = sf * (np.arange(4) - zf)
            for k in range(128 * g, 128 * g + 128):
                err = np.abs(float(W[n, k]) - levels)
                o = np.argsort(err)
                if err[o[1]] - err[o[0]] > 1e-9:
                    assert q[n, k] == o[0]


@pytest.mark.parametrize("val", [0.0, 1e-9, -0.3, 0.7])
def test_int2_degenerate_groups(val):
    # constant groups: the range [min(v,0), max(v,0)] puts v on a level (up
    # to the fp16 rounding of s); a scale that underflows is stored as 1 and
    # the group dequantizes to 0
    W = np.full((1, 128), val, np.float32)
    q, s, z, w = _int2_roundtrip(W)
    assert s[0, 0] != 0
    if abs(val) < 1e-6:
        assert s[0, 0] == 1 and np.all(w == 0)
    else:
        assert np.max(np.abs(w - W)) <= 3 * 2.0 ** -11 * abs(val)


def test_int2_pack_layout():
    q = np.zeros((1, 32), np.uint8)
    q[0, 17] = 3                           # word 1, field 1 -> bits 2..3
    words = pack.pack_int2(q)
    assert words.tolist() == [[0, 3 << 2]]
    assert np.array_equal(pack.unpack_int2(words, 32), q)


# ---- int3 g128 (Whetstone, "int3 g128": 3-bit codes, int4-style metadata) ----

def _int3_roundtrip(W):
    q, s, z = quant.quantize_int3_g128(W)
    codes = pack.pack_int3(q)
    return q, s, z, codes, ref.dequant_int3(codes, pack.pack_int4_meta(s, z), W.shape[1])


def test_int3_lossless_on_grid():
    # weights on the 1/8 grid spanning [-0.5, 0.375]: hi - lo = 7/8, s = 1/8,
    # z = 4 and q = 8 w + 4
    k = np.tile(np.arange(8), 16)
    W = ((k.astype(np.float32) - 4) / np.float32(8))[None, :]
    q, s, z, codes, w = _int3_roundtrip(W)
    assert s[0, 0] == np.float16(0.125) and z[0, 0] == 4
    assert np.array_equal(q[0].astype(int), k)
    assert np.array_equal(w.astype(np.float32), W)


def test_int3_codes_are_nearest_level():
    rng = np.random.default_rng(31)
    W = (rng.standard_normal((4, 256)) * 0.02).astype(np.float32)
    q, s, z, codes, w = _int3_roundtrip(W)
    for n in range(4):
        for g in range(2):
            levels = float(s[n, g]) * (np.arange(8) - float(z[n, g]))
            for k in range(128 * g, 128 * g + 128):
                err = np.abs(float(W[n, k]) - levels)
                o = np.argsort(err)
                if err[o[1]] - err[o[0]] > 1e-9:
                    assert q[n, k] == o[0]


def test_int3_layout_one_hot():
    """Each code position lands where the layout text puts it (row 1 of a
    3-row matrix, so a row-major plane order would put it elsewhere)."""
    K, N, n = 256, 3, 1
    for pos, val in [(0, 7), (4, 5), (5, 3), (9, 7), (10, 1), (27, 6), (29, 7), (30, 5), (31, 6),
                     (128 + 32 * 3 + 31, 7), (128 + 64 + 17, 2)]:
        q = np.zeros((N, K), np.uint8)
        q[n, pos] = val
        words = pack.pack_int3(q)
        assert words.shape == (3, N, K // 32)
        flat = words.reshape(-1)
        g, e = divmod(pos, 128)
        b, t = divmod(e, 32)
        widx = 3 * b                           # index of W0 of the block in the group's 12 words
        nz = np.flatnonzero(flat)

        def word_index(i):                     # word i of the group: plane i // 4, word i % 4
            return ((i // 4) * N + n) * (K // 32) + 4 * g + i % 4

        expect = {}
        if t < 30:
            j, f = divmod(t, 10)
            shift = 3 * f if f < 5 else 16 + 3 * (f - 5)
            expect[word_index(widx + j)] = val << shift
        else:
            for j in range(3):
                if (val >> j) & 1:
                    expect[word_index(widx + j)] = 1 << (15 if t == 30 else 31)
        assert sorted(nz.tolist()) == sorted(expect), pos
        for idx, v in expect.items():
            assert int(flat[idx]) == v, pos
        assert np.array_equal(pack.unpack_int3(words, K), q)


def test_int3_roundtrip_random_codes():
    q = np.random.default_rng(32).integers(0, 8, (5, 384)).astype(np.uint8)
    assert np.array_equal(pack.unpack_int3(pack.pack_int3(q), 384), q)

"""Pins of the packers and unpackers: round trips, and one-hot codes placed in
each slot giving the word value the layout text dictates."""

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import pack


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 4), st.integers(1, 4), st.integers(0, 2**32 - 1))
def test_int4_round_trip(n, kw, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, (n, 8 * kw)).astype(np.uint8)
    w = pack.pack_int4(q)
    assert w.dtype == np.uint32 and w.shape == (n, kw)
    assert np.array_equal(pack.unpack_int4(w, 8 * kw), q)


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 4), st.integers(1, 3), st.integers(0, 2**32 - 1))
def test_tern_and_bits_round_trip(n, kw, seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 3, (n, 16 * kw)).astype(np.uint8)
    assert np.array_equal(pack.unpack_tern(pack.pack_tern(c), 16 * kw), c)
    b = rng.integers(0, 2, (n, 32 * kw)).astype(np.uint8)
    assert np.array_equal(pack.unpack_bits(pack.pack_bits(b), 32 * kw), b)


def test_int4_one_hot_slots():
    for i in range(8):
        for v in (1, 9, 15):
            q = np.zeros((1, 16), np.uint8)
            q[0, 8 + i] = v          # second word, slot i
            w = pack.pack_int4(q)
            assert w[0, 0] == 0
            assert int(w[0, 1]) == v << (4 * i)


def test_int4_extremes():
    assert np.all(pack.pack_int4(np.zeros((2, 8), np.uint8)) == 0)
    assert np.all(pack.pack_int4(np.full((2, 8), 15, np.uint8)) == 0xFFFFFFFF)
    # element order: nibble i of word j is element 8j+i
    q = np.arange(8, dtype=np.uint8)[None, :]
    assert int(pack.pack_int4(q)[0, 0]) == 0x76543210


def test_tern_and_bits_slots():
    for i in range(16):
        c = np.zeros((1, 16), np.uint8)
        c[0, i] = 2
        assert int(pack.pack_tern(c)[0, 0]) == 2 << (2 * i)
    for i in range(32):
        b = np.zeros((1, 32), np.uint8)
        b[0, i] = 1
        assert int(pack.pack_bits(b)[0, 0]) == 1 << i


def test_meta_half2_layout():
    s = np.array([[1.0, 0.5]], np.float16)
    z = np.array([[3.0, 15.0]], np.float16)
    m = pack.pack_int4_meta(s, z)
    # fp16 1.0 = 0x3C00, 3.0 = 0x4200, 0.5 = 0x3800, 15.0 = 0x4B80
    assert int(m[0, 0]) == 0x42003C00
    assert int(m[0, 1]) == 0x4B803800
    s2, z2 = pack.unpack_int4_meta(m)
    assert np.array_equal(s2, s) and np.array_equal(z2, z)

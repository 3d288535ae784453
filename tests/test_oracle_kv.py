"""Pins of oracle.kv (the low-bit KV-cache decode attention oracle; the
BitDecoding README's usage: 4-bit codes, group 128, K per channel, V per
token, head dimension 128): closed forms of single-query softmax attention,
its shift invariance, the GQA head mapping, lossless pages on a grid, and the
page layout position by position."""

import numpy as np
import pytest

from oracle import kv, pack


def _grid_page(rng):
    """K and V pages whose groups are exactly representable: every K channel
    (over the page's tokens) and every V token (over its channels) spans
    [-8/16, 7/16] on the 1/16 grid."""
    def rows(n):
        r = rng.integers(0, 16, (n, 128))
        r[:, 0], r[:, 1] = 0, 15
        return (r.astype(np.float32) - 8) / np.float32(16)
    Kp = rows(128).T.copy()          # per channel = rows of K^T
    Vp = rows(128)                   # per token = rows of V
    return Kp, Vp


def test_page_lossless_on_grid():
    Kp, Vp = _grid_page(np.random.default_rng(40))
    words = kv.pack_page(*kv.quantize_page(Kp, Vp))
    K, V = kv.unpack_page(words)
    assert np.array_equal(K, Kp.astype(np.float64)) and np.array_equal(V, Vp.astype(np.float64))
    ks, kz = pack.unpack_int4_meta(words[4096:4224])
    assert np.all(ks == np.float16(1 / 16)) and np.all(kz == 8)


def test_page_layout_positions():
    kc = np.zeros((128, 128), np.uint8)
    vc = np.zeros((128, 128), np.uint8)
    kc[5, 13] = 9        # token 5, channel 13 -> K word 5*16 + 1, bits 4*5
    vc[70, 3] = 6        # token 70, channel 3 -> V word 2048 + 3*16 + 8, bits 4*6
    one = np.ones(128, np.float16)
    zero = np.zeros(128, np.float16)
    w = kv.pack_page(kc, one, zero, vc, one * 2, zero + 3)
    nz = np.flatnonzero(w[:4096])
    assert nz.tolist() == [5 * 16 + 1, 2048 + 3 * 16 + 8]
    assert w[5 * 16 + 1] == 9 << 20 and w[2048 + 3 * 16 + 8] == 6 << 24
    assert np.all(w[4096:4224] == 0x00003C00) and np.all(w[4224:4352] == 0x42004000)
    K, V = kv.unpack_page(w)
    assert K[5, 13] == 9 and np.count_nonzero(K) == 1
    assert V[70, 3] == 2 * (6 - 3) and V[0, 0] == 2 * (0 - 3)


def test_attention_uniform_scores_is_mean():
    rng = np.random.default_rng(41)
    K = rng.standard_normal((1, 2, 256, 128))
    V = rng.standard_normal((1, 2, 256, 128))
    q = np.zeros((1, 2, 128))
    out, p = kv.attention_decode(q, K, V, 0.1)
    assert np.allclose(p, 1 / 256, rtol=0, atol=1e-15)
    assert np.allclose(out[0, 1], V[0, 1].mean(axis=0), rtol=0, atol=1e-12)


def test_attention_dominant_token():
    rng = np.random.default_rng(42)
    K = rng.standard_normal((1, 1, 128, 128)) * 0.01
    V = rng.standard_normal((1, 1, 128, 128))
    K[0, 0, 77] = 1.0
    q = np.ones((1, 1, 128))
    out, p = kv.attention_decode(q, K, V, 1.0)      # score 128 vs ~0
    assert p[0, 0].argmax() == 77 and p[0, 0, 77] >= 1 - 1e-12
    assert np.allclose(out[0, 0], V[0, 0, 77], atol=1e-12)


def test_attention_shift_invariance():
    # adding c * q / |q|^2 / scale to every key shifts every score by c
    rng = np.random.default_rng(43)
    K = rng.standard_normal((1, 1, 128, 128))
    V = rng.standard_normal((1, 1, 128, 128))
    q = rng.standard_normal((1, 1, 128))
    sc = 1 / np.sqrt(128)
    a, _ = kv.attention_decode(q, K, V, sc)
    b, _ = kv.attention_decode(q, K + 3.0 * q[0, 0] / (q[0, 0] @ q[0, 0]) / sc, V, sc)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_gqa_head_mapping():
    # KV head j carries the constant value j + 1: query head h must read h // 4
    K = np.zeros((1, 2, 128, 128))
    V = np.stack([np.full((128, 128), 1.0), np.full((128, 128), 2.0)])[None]
    q = np.random.default_rng(44).standard_normal((1, 8, 128))
    out, _ = kv.attention_decode(q, K, V, 1.0)
    assert np.allclose(out[0, :4], 1.0) and np.allclose(out[0, 4:], 2.0)


def test_cache_roundtrip_and_bound_shape():
    rng = np.random.default_rng(45)
    K = (rng.standard_normal((1, 256, 2, 128))).astype(np.float16)
    V = (rng.standard_normal((1, 256, 2, 128))).astype(np.float16)
    cache = kv.pack_cache(K, V)
    assert cache.shape == (1, 2, 2, kv.PAGE_WORDS) and kv.PAGE_BYTES == 17408
    Kd, Vd = kv.dequant_cache(cache)
    # 4-bit per-group quantization: within half a step (+ fp16 scale rounding)
    for p in range(2):
        sl = slice(128 * p, 128 * p + 128)
        kp = K[0, sl, 1].astype(np.float64)
        step = (np.maximum(kp.max(0), 0) - np.minimum(kp.min(0), 0)) / 15
        assert np.all(np.abs(Kd[0, 1, sl] - kp) <= step[None, :] * 0.51 + 1e-3)
    q = rng.standard_normal((1, 4, 128))
    b = kv.attention_bound(q, Kd, Vd, 1 / np.sqrt(128))
    assert b.shape == (1, 4, 128) and np.all(b > 0)
    with pytest.raises(ValueError):
        kv.pack_cache(K[:, :100], V[:, :100])

"""Pins of oracle.kv (the low-bit KV-cache decode attention oracle; the
BitDecoding README's usage: 4-bit codes, group 128, K per channel, V per
token, head dimension 128): closed forms of single-query softmax attention,
its shift invariance, the GQA head mapping, lossless pages on a grid, the
page layout position by position, and the tolerance: its closed form when
every score ties, worst-case perturbations inside the two per-GEMV budgets
(which must stay inside it and come close to it), and a dropped or repeated
page, which it must reject at 4096, 32768 and 131072 cached tokens."""

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
from oracle import kv, pack
from oracle.ref import TOL


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
    # bounded below by the value GEMV's own budget, eps * sum_t p_t |V_tc|
    _, pr = kv.attention_decode(q, Kd, Vd, 1 / np.sqrt(128))
    assert np.all(b[0, 0] >= TOL * (pr[0, 0] @ np.abs(Vd[0, 0])))
    with pytest.raises(ValueError):
        kv.pack_cache(K[:, :100], V[:, :100])


def test_bound_closed_form_when_scores_tie():
    # K = 0: every A_t is 0, so the bound is eps * sum_t p_t |V_tc| = eps * mean_t |V_tc|
    rng = np.random.default_rng(46)
    K = np.zeros((1, 1, 384, 128))
    V = rng.standard_normal((1, 1, 384, 128))
    q = rng.standard_normal((1, 2, 128))
    b = kv.attention_bound(q, K, V, 0.3)
    assert np.allclose(b[0, 0], TOL * np.abs(V[0, 0]).mean(axis=0), rtol=1e-12, atol=0)
    assert np.array_equal(b[0, 0], b[0, 1])


def _perturbed(q, K, V, sm_scale, c, sign_s, sign_v):
    """Attention with every score moved by sign_s[t] * eps * A_t and the value
    product moved by sign_v * eps * sum_t p'_t |V_tc| (channel c)."""
    s = sm_scale * (K @ q)
    A = sm_scale * (np.abs(K) @ np.abs(q))
    s2 = s + sign_s * TOL * A
    e = np.exp(s2 - s2.max())
    p2 = e / e.sum()
    return p2 @ V[:, c] + sign_v * TOL * (p2 @ np.abs(V[:, c]))


def test_bound_holds_and_is_tight_under_worst_perturbations():
    rng = np.random.default_rng(47)
    sm = 1 / np.sqrt(128)
    worst = 0.0
    for trial in range(6):
        T = 128 * (1 + trial)
        K = rng.standard_normal((T, 128)) * (0.5 + trial)
        V = rng.standard_normal((T, 128))
        q = rng.standard_normal(128)
        ref, p = kv.attention_decode(q[None, None], K[None, None], V[None, None], sm)
        bound = kv.attention_bound(q[None, None], K[None, None], V[None, None], sm, probs=p)[0, 0]
        for c in range(0, 128, 9):
            for direction in (1.0, -1.0):
                # push probability towards the tokens that move channel c in `direction`
                sign_s = np.where((V[:, c] - ref[0, 0, c]) * direction > 0, 1.0, -1.0)
                got = _perturbed(q, K, V, sm, c, sign_s, direction)
                err = abs(got - ref[0, 0, c])
                assert err <= bound[c] * (1 + 1e-9), (trial, c, err / bound[c])
                worst = max(worst, err / bound[c])
        # random perturbations inside the budgets stay inside too
        for _ in range(20):
            got = _perturbed(q, K, V, sm, 5, rng.uniform(-1, 1, T), rng.uniform(-1, 1))
            assert abs(got - ref[0, 0, 5]) <= bound[5]
    # the derivation is not loose by orders of magnitude: the worst case
    # reaches a large part of it
    assert worst > 0.3, worst


@pytest.mark.parametrize("T", [4096, 32768, 131072])
def test_bound_rejects_a_dropped_or_repeated_page(T):
    """Page-marker cache (every score ties; the marker channel of page p is
    (p + 0) % 128): the exact attention passes its own check; the same
    attention with one page left out, or with one page's content read twice
    in place of another's, fails it."""
    K, V, q = inputs.kv_marker_case(1, 1, 1, T)
    cache = kv.pack_cache(K, V)
    Kd, Vd = kv.dequant_cache(cache)
    assert np.array_equal(Vd[0, 0], V[0, :, 0].astype(np.float64))     # exact on the grid
    sm = 1 / np.sqrt(128)
    qd = q.astype(np.float64)
    ref, p = kv.attention_decode(qd, Kd, Vd, sm)
    bound = kv.attention_bound(qd, Kd, Vd, sm, probs=p)
    assert np.all(np.abs(ref - ref) <= bound)
    P = T // 128
    for j in sorted({0, 1, P // 2, P - 2, P - 1}):
        keep = np.ones(T, bool)
        keep[128 * j:128 * (j + 1)] = False
        dropped, _ = kv.attention_decode(qd, Kd[:, :, keep], Vd[:, :, keep], sm)
        assert np.any(np.abs(dropped - ref) > bound), "page %d dropped passes" % j
        i = (j + 1) % P
        Vr = Vd.copy()
        Vr[:, :, 128 * i:128 * (i + 1)] = Vd[:, :, 128 * j:128 * (j + 1)]
        repeated, _ = kv.attention_decode(qd, Kd, Vr, sm)
        assert np.any(np.abs(repeated - ref) > bound), "page %d read twice passes" % j


def test_lengths_equal_truncation():
    """Attention over the first lens[b] tokens is attention over the cache cut
    to those tokens; probabilities past the length are 0; full lengths are
    the plain case; a sequence of length 0 has output 0."""
    rng = np.random.default_rng(48)
    K = rng.standard_normal((3, 2, 384, 128))
    V = rng.standard_normal((3, 2, 384, 128))
    q = rng.standard_normal((3, 4, 128))
    lens = [300, 129, 0]
    out, p = kv.attention_decode(q, K, V, 0.1, lens)
    for b, n in enumerate(lens[:2]):
        ref, pr = kv.attention_decode(q[b:b + 1], K[b:b + 1, :, :n], V[b:b + 1, :, :n], 0.1)
        assert np.allclose(out[b], ref[0], rtol=0, atol=1e-12)
        assert np.allclose(p[b, :, :n], pr[0], rtol=0, atol=1e-15) and not p[b, :, n:].any()
    assert not out[2].any() and not p[2].any()
    full, _ = kv.attention_decode(q, K, V, 0.1)
    assert np.array_equal(kv.attention_decode(q, K, V, 0.1, [384] * 3)[0], full)
    b = kv.attention_bound(q, K, V, 0.1, lens=lens)
    assert not b[2].any() and np.all(b[:2] > 0)


def test_partial_page_quantizes_its_valid_tokens_only():
    """Sequence of 200 tokens in a 256-token cache: in page 1 (72 valid
    tokens) every K channel's scale and zero-point are those of the valid
    tokens alone (the group range spans 0 either way), the tokens past the
    length are zero V groups (scale 1, zero 0, codes 0), and page 0 is the
    same as without lengths."""
    rng = np.random.default_rng(49)
    K = rng.standard_normal((1, 256, 1, 128)).astype(np.float16)
    V = rng.standard_normal((1, 256, 1, 128)).astype(np.float16)
    cache = kv.pack_cache(K, V, [200])
    assert np.array_equal(cache[0, 0, 0], kv.pack_cache(K, V)[0, 0, 0])
    page = cache[0, 0, 1]
    ks, kz = pack.unpack_int4_meta(page[4096:4224])
    v = K[0, 128:200, 0].astype(np.float32)
    lo = np.minimum(v.min(axis=0), 0)
    hi = np.maximum(v.max(axis=0), 0)
    s = ((hi - lo) / np.float32(15)).astype(np.float16)
    assert np.array_equal(ks, s) and np.array_equal(kz, np.clip(np.rint(-lo / s.astype(np.float32)), 0, 15))
    vs, vz = pack.unpack_int4_meta(page[4224:4352])
    assert np.all(vs[72:] == 1) and np.all(vz[72:] == 0)
    Kd, Vd = kv.unpack_page(page)
    assert not Vd[72:].any() and not Kd[72:].any()


def test_bound_rejects_a_dropped_partial_page():
    """Page markers with a sequence of 1000 tokens in a 1024-token cache: the
    exact attention passes; leaving out the last, partial page (104 valid
    tokens) or reading the page before it in its place fails."""
    K, V, q = inputs.kv_marker_case(1, 1, 1, 1024)
    cache = kv.pack_cache(K, V, [1000])
    Kd, Vd = kv.dequant_cache(cache)
    sm = 1 / np.sqrt(128)
    qd = q.astype(np.float64)
    ref, p = kv.attention_decode(qd, Kd, Vd, sm, [1000])
    bound = kv.attention_bound(qd, Kd, Vd, sm, probs=p, lens=[1000])
    dropped, _ = kv.attention_decode(qd, Kd, Vd, sm, [896])
    assert np.any(np.abs(dropped - ref) > bound)
    Vr = Vd.copy()
    Vr[:, :, 896:1024] = Vd[:, :, 768:896]
    repeated, _ = kv.attention_decode(qd, Kd, Vr, sm, [1000])
    assert np.any(np.abs(repeated - ref) > bound)

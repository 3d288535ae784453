"""Pins of the int4-hier-g32 oracle (quantizer, metadata layout, dequant,
accounting).

The pages fix the format's cost (Whetstone: 4.28 bits/weight, ~0.03 above
int4 g128, 264.4 MB per 0.5B token) and its structure (two 4-bit indices per
32-group against one fp16 pair per row, like Q4_K); the quantizer is the
round-to-nearest reading in oracle.quant.  Pins: the page's byte figures
from the layout, lossless round trips on constructed grids, brute-force
optimality of every rounding step on small rows, the row-scale underflow
guard, and a closed-form dequantization.
"""

import os

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
from oracle import accounting as acc
from oracle import pack, quant, ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    vals = {}
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#") and not line.startswith("fmt"):
            k, v = line.split()[:2]
            vals[k] = float(v)
    return vals


def _roundtrip(W):
    q, sc, mi, d16, dmin16 = quant.quantize_int4_hier_g32(W)
    N, K = W.shape
    codes = pack.pack_int4(q)
    meta = pack.pack_hier_meta(sc, mi, d16, dmin16)
    return (q, sc, mi, d16, dmin16), codes, meta, ref.dequant_int4_hier(codes, meta, N, K)


def test_accounting_matches_page():
    vals = _gold("metadata_bits.txt")
    shapes = inputs.sweep_shapes("qwen2.5-0.5b")
    params = acc.linear_params(shapes)
    hier = sum(acc.weight_bytes("hier", n, k) for _, n, k in shapes)
    g128 = sum(acc.weight_bytes("int4", n, k) for _, n, k in shapes)
    bpw = 8.0 * hier / params
    assert round(bpw, 2) == vals["int4_hier_g32_bpw"]
    assert round(bpw - 8.0 * g128 / params, 2) == vals["hier_g32_extra_bpw"]
    assert abs(hier / 1e6 - 264.4) <= 0.2          # bytes/token table row
    # per matrix: K/2 + K/32 bytes per row plus one 4-byte pair per row
    assert acc.weight_bytes("hier", 896, 896) == 896 * 448 + 896 * 28 + 896 * 4


def test_meta_layout_one_hot():
    N, K = 3, 96
    sc = np.zeros((N, 3), np.uint8)
    mi = np.zeros((N, 3), np.uint8)
    sc[2, 1], mi[1, 2] = 7, 9
    d16 = np.array([1.0, 2.0, 0.5], np.float16)
    dmin16 = np.array([0.25, -0.0, 3.0], np.float16)
    blk = pack.pack_hier_meta(sc, mi, d16, dmin16)
    R = pack.hier_row_offset(N, K)
    assert R == 16 and blk.size == R + 12
    assert blk[2 * 3 + 1] == 7 and blk[1 * 3 + 2] == 9 << 4
    assert np.count_nonzero(blk[:R]) == 2
    rows = blk[R:].view("<u4")
    assert rows[1] == (np.float16(2.0).view(np.uint16) | (np.float16(-0.0).view(np.uint16).astype(np.uint32) << 16))
    back = pack.unpack_hier_meta(blk, N, K)
    assert np.array_equal(back[0], sc) and np.array_equal(back[1], mi)
    assert np.array_equal(back[2].view(np.uint16), d16.view(np.uint16))
    assert np.array_equal(back[3].view(np.uint16), dmin16.view(np.uint16))


def test_dequant_closed_form():
    # one row, one group: d = 0.5, dmin = 0.25, sc = 3, mi = 2 -> w = 1.5 q - 0.5
    q = np.arange(32, dtype=np.uint8)[None, :] % 16
    meta = pack.pack_hier_meta(np.array([[3]], np.uint8), np.array([[2]], np.uint8),
                               np.array([0.5], np.float16), np.array([0.25], np.float16))
    w = ref.dequant_int4_hier(pack.pack_int4(q), meta, 1, 32)
    assert np.array_equal(w[0], 1.5 * (np.arange(32) % 16) - 0.5)


def _grid_matrix(rng, N, ng):
    """Weights exactly on a chosen hierarchical grid, built so that RTN must
    recover the chosen codes: every group holds codes 0 and 15 (its range is
    exactly 15 steps), one group of each row has sc = 15 and one has mi = 15
    (the row maxima give back d and dmin), and the top of every group is
    >= 0 (the range widened to 0 is the group's own range)."""
    d = np.float16(2.0 ** -7)
    dmin = np.float16(2.0 ** -8)
    sc = rng.integers(1, 16, (N, ng))
    mi = rng.integers(0, 16, (N, ng))
    sc[:, 0], mi[:, 1] = 15, 15
    mi = np.minimum(mi, (15 * float(d) * sc / float(dmin)).astype(int))  # top >= 0
    mi[:, 1] = 15
    sc[:, 1] = np.maximum(sc[:, 1], 8)   # 15 d sc >= 15 dmin: needs sc >= 8 here
    q = rng.integers(0, 16, (N, ng, 32))
    q[:, :, 0], q[:, :, 1] = 0, 15
    W = float(d) * sc[:, :, None] * q - float(dmin) * mi[:, :, None]
    return W.reshape(N, ng * 32).astype(np.float32), q.reshape(N, ng * 32), sc, mi, d, dmin


def test_lossless_on_grid():
    rng = np.random.default_rng(11)
    W, q0, sc0, mi0, d0, dmin0 = _grid_matrix(rng, 5, 7)
    (q, sc, mi, d16, dmin16), codes, meta, w = _roundtrip(W)
    assert np.all(d16 == d0) and np.all(dmin16 == dmin0)
    assert np.array_equal(sc, sc0) and np.array_equal(mi, mi0)
    assert np.array_equal(q.astype(int), q0)
    assert np.array_equal(w, W.astype(np.float64))


def test_every_rounding_step_is_nearest():
    """Brute force on small rows: each stored index / code is the nearest
    admissible one to the quantity it approximates (ties excluded)."""
    rng = np.random.default_rng(12)
    W = (rng.standard_normal((6, 128)) * 0.02).astype(np.float32)
    W[1] += 0.01                                      # lopsided rows too
    W[2] -= 0.03
    (q, sc, mi, d16, dmin16), codes, meta, w = _roundtrip(W)
    G = W.astype(np.float64).reshape(6, 4, 32)
    lo = np.minimum(G.min(2), 0)
    hi = np.maximum(G.max(2), 0)
    s, m = (hi - lo) / 15, -lo
    for n in range(6):
        d, dm = float(d16[n]), float(dmin16[n])
        assert abs(d - s[n].max() / 15) <= 2.0 ** -11 * s[n].max() / 15 * 1.01
        assert abs(dm - m[n].max() / 15) <= 2.0 ** -11 * m[n].max() / 15 * 1.01
        for g in range(4):
            cand = np.abs(s[n, g] - d * np.arange(1, 16))
            best = np.argsort(cand)
            if cand[best[1]] - cand[best[0]] > 1e-9:
                assert sc[n, g] == best[0] + 1
            cand = np.abs(m[n, g] - dm * np.arange(16))
            best = np.argsort(cand)
            if cand[best[1]] - cand[best[0]] > 1e-9:
                assert mi[n, g] == best[0]
            step, off = d * sc[n, g], dm * mi[n, g]
            for k in range(32):
                err = np.abs(G[n, g, k] - (step * np.arange(16) - off))
                best = np.argsort(err)
                if err[best[1]] - err[best[0]] > 1e-9:
                    assert q[n, 32 * g + k] == best[0]
    # and the dequantized weight is within half a step of every unclipped weight
    step = np.repeat(d16.astype(np.float64)[:, None] * sc, 32, axis=1)
    inside = (q > 0) & (q < 15)
    assert np.all(np.abs(w - W)[inside] <= step[inside] / 2 * (1 + 1e-6))


@pytest.mark.parametrize("val", [0.0, 1e-9, -1e-9, 3e-8])
def test_row_scale_underflow_guard(val):
    """Whetstone, status list: a row scale that underflows fp16 must not turn
    the row into garbage.  Tiny rows store d = 1 (and/or dmin = 1) and
    dequantize to within their own magnitude."""
    W = np.full((2, 64), val, np.float32)
    W[1, ::3] = -val
    (q, sc, mi, d16, dmin16), codes, meta, w = _roundtrip(W)
    assert np.all(d16 != 0) and np.all(dmin16 != 0)
    assert np.all(np.isfinite(w))
    assert np.max(np.abs(w - W)) <= 2 * abs(val) + 1e-12
    if val == 0.0:
        assert np.all(w == 0) and np.all(d16 == 1) and np.all(dmin16 == 1)


def test_tiny_row_beside_normal_row():
    # a per-row scale: a tiny row keeps its own precision next to a large one
    rng = np.random.default_rng(13)
    W = (rng.standard_normal((2, 256)) * 0.02).astype(np.float32)
    W[1] *= np.float32(1e-3)
    _, _, _, w = _roundtrip(W)
    for n in range(2):
        rel = np.linalg.norm(w[n] - W[n]) / np.linalg.norm(W[n])
        assert rel < 0.12


def test_finer_than_g128_on_gaussian_rows():
    """Whetstone, quantizer table: group 32 with hierarchical metadata loses
    less than group 128.  On N(0, 0.02) rows the weight error must drop."""
    rng = np.random.default_rng(14)
    W = (rng.standard_normal((64, 896)) * 0.02).astype(np.float32)
    _, _, _, wh = _roundtrip(W)
    q, s, z = quant.quantize_int4_g128(W)
    wg = ref.dequant_int4(pack.pack_int4(q), pack.pack_int4_meta(s, z), 896)
    eh = np.linalg.norm(wh - W) / np.linalg.norm(W)
    eg = np.linalg.norm(wg - W) / np.linalg.norm(W)
    assert eh < 0.9 * eg


def test_shape_validation():
    with pytest.raises(ValueError):
        quant.quantize_int4_hier_g32(np.zeros((2, 48), np.float32))

"""C-ABI checks that need no GPU: the library loads, exports every function
include/tkq.h declares, its structs have the declared layout, argument
validation rejects bad calls before any HIP call, and the GEMV planner's
host-side output is consistent."""

import ctypes
import os
import re

import pytest

from gemm_tkq_gemv_amd import inputs, tkq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tkq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tkq.LIB_PATH), reason="libtkq.so not built")

A = 0x7f0000000000  # fake, 16-byte aligned device addresses (never dereferenced)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tkq_\w+)\s*\(", text)))


def test_exports_every_declared_function():
    names = _declared()
    assert "tkq_gemv" in names and "tkq_gemm_prefill" in names
    lib = tkq.lib()
    for name in names:
        assert hasattr(lib, name), name
    # and the binding types every one of them
    assert set(names) == set(tkq._SIGNATURES)


def test_struct_layout():
    assert ctypes.sizeof(tkq.GemvDesc) == 64
    assert ctypes.sizeof(tkq.GemvPlan) == 32
    assert tkq.GemvDesc.codes.offset == 32 and tkq.GemvDesc.y.offset == 56
    text = open(HEADER).read()
    assert "} tkq_gemv_desc;         /* 64 bytes */" in text


def test_version_and_strings():
    lib = tkq.lib()
    assert lib.tkq_version() == 10000
    for st in range(0, -7, -1):
        assert tkq.strerror(st)
    assert "unknown" in tkq.strerror(-99)


@pytest.mark.parametrize("name", ["tkq_pack_int4_g128", "tkq_pack_k5", "tkq_pack_tern_g128",
                                  "tkq_pack_int4_hier_g32", "tkq_pack_int2_g128", "tkq_pack_int3_g128"])
def test_pack_validation(name):
    f = getattr(tkq.lib(), name)
    assert f(None, 4, 128, A, A, None) == tkq.EINVAL
    assert f(A, 0, 128, A, A, None) == tkq.EINVAL
    assert f(A, 4, 0, A, A, None) == tkq.EINVAL
    assert f(A, 4, 100, A, A, None) == tkq.ESHAPE
    if name != "tkq_pack_int4_hier_g32":
        assert f(A, 4, 96, A, A, None) == tkq.ESHAPE   # group 128
    assert f(A, 4, 48, A, A, None) == tkq.ESHAPE
    assert f(A, 4, (1 << 20) + 128, A, A, None) == tkq.ESHAPE
    assert f(A, 1 << 31, 128, A, A, None) == tkq.ESHAPE
    assert f(A, 4, 128, None, A, None) == tkq.EINVAL
    assert f(A, 4, 128, A, None, None) == tkq.EINVAL
    assert f(A + 4, 4, 128, A, A, None) == tkq.EALIGN
    assert f(A, 4, 128, A + 8, A, None) == tkq.EALIGN
    assert f(A, 4, 128, A, A + 2, None) == tkq.EALIGN


def test_hier_meta_bytes():
    f = tkq.lib().tkq_hier_meta_bytes
    assert f(1, 32) == 16 + 4                      # one group byte, padded to 16
    assert f(896, 896) == 896 * 28 + 4 * 896       # 25088 is a multiple of 16
    assert f(3, 96) == 16 + 12
    assert f(5, 160) == 32 + 20                    # 25 group bytes -> 32
    assert f(0, 32) == -1 and f(4, 48) == -1 and f(4, 0) == -1
    from oracle import pack as opack
    for n, k in [(1, 32), (3, 96), (5, 160), (151936, 896), (3584, 18944)]:
        assert f(n, k) == opack.hier_meta_bytes(n, k)


def test_pack_bin_validation():
    f = tkq.lib().tkq_pack_bin
    assert f(None, 1, 32, A, None) == tkq.EINVAL
    assert f(A, 1, 48, A, None) == tkq.ESHAPE
    assert f(A, 1, 32, None, None) == tkq.EINVAL
    assert f(A, 1, 32, A + 4, None) == tkq.EALIGN


def _descs(fmt, shapes):
    arr = (tkq.GemvDesc * len(shapes))()
    for i, (n, k) in enumerate(shapes):
        d = arr[i]
        d.fmt, d.N, d.K = fmt, n, k
        d.codes, d.meta, d.x, d.y = A, A + 0x100000, A + 0x200000, A + 0x300000
    return arr


def _prepare(arr):
    plan = tkq.GemvPlan()
    st = tkq.lib().tkq_gemv_prepare(arr, len(arr), ctypes.byref(plan))
    return st, plan


def _shape(d):
    return 1 << (d.shape & 15), (d.shape >> 4) & 4095, (d.shape >> 16) & 15


def _tiles(d):
    """Row ranges of a prepared descriptor's tiles: large, then small."""
    out, r = [], 0
    for _ in range(d.big_tiles):
        out.append((r, d.rows_per_tile))
        r += d.rows_per_tile
    while r < d.N:
        out.append((r, d.small_rows))
        r += d.small_rows
    return out


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5, 6, 7])
def test_prepare_tiles_cover_rows(fmt):
    shapes = [(1, 128), (7, 896), (128, 896), (4864, 896), (896, 4864), (333, 4864), (151936, 896)]
    if fmt == 5:
        shapes[1:1] = [(3, 32), (65, 96)]
    arr = _descs(fmt, shapes)
    st, plan = _prepare(arr)
    assert st == tkq.OK
    work = 0
    per_chunk = {1: 32, 2: 16, 3: 64, 4: 128, 5: 32, 6: 64, 7: 128}[fmt]
    for d, (n, k) in zip(arr, shapes):
        assert d.work0 == work
        tiles = _tiles(d)
        # tiles are disjoint, in order, and cover rows 0..N-1 (the last may overhang)
        assert tiles[0][0] == 0 and tiles[-1][0] < n <= tiles[-1][0] + tiles[-1][1]
        for (r0, h0), (r1, _) in zip(tiles, tiles[1:]):
            assert r1 == r0 + h0
        L, J, S = _shape(d)
        C = k // per_chunk
        if fmt == 1:
            # int4: 32 units of R rows per tile, R even when a row has an odd
            # number of 128-weight groups (unless R = 1)
            assert (L, J, S) == (8, k // 128, 1)
            for h in (d.rows_per_tile, d.small_rows):
                assert h % 32 == 0 and 0 < h <= 1024
                assert (k // 128) % 2 == 0 or h == 32 or h % 64 == 0
            assert d.small_rows <= d.rows_per_tile
            work += len(tiles)
            continue
        assert S in (1, 2, 4) and 1 <= J <= 8
        assert S * L * J >= C                       # every chunk has a lane
        P = 64 // L
        for h in (d.rows_per_tile, d.small_rows):
            assert h % ((4 // S) * P) == 0 and 0 < h <= 1024
        assert d.small_rows <= d.rows_per_tile
        work += len(tiles)
    assert plan.tiles == work and plan.count == len(shapes) and plan.fmt == fmt
    # the last stretch of a long sweep is cut into small tiles
    last = arr[len(shapes) - 1]
    assert last.big_tiles * last.rows_per_tile < last.N


def test_tile_edge_rows_match_the_plan():
    """The GPU sweep test checks the first and last row of every tile through
    helpers.tile_edge_rows: on the 7B plan it must name exactly the edges of
    the tiles the planner made."""
    from helpers import tile_edge_rows
    shapes = [(n, k) for _, n, k in inputs.sweep_shapes("qwen2.5-7b")]
    arr = _descs(1, shapes)
    assert _prepare(arr)[0] == tkq.OK
    for d in arr:
        want = set()
        for r0, h in _tiles(d):
            want |= {r0, min(d.N, r0 + h) - 1}
        assert set(tile_edge_rows(d).tolist()) == want


def test_prepare_shapes_for_model_matrices():
    arr = _descs(1, [(896, 896), (896, 4864), (3584, 3584), (3584, 18944)])
    assert _prepare(arr)[0] == tkq.OK
    # int4: units of eight lanes, the pass field holds the row's group count
    assert [_shape(d) for d in arr] == [(8, 7, 1), (8, 38, 1), (8, 28, 1), (8, 148, 1)]
    # rows per tile: 32 units of R rows, R from 48 KB per wave (even for 7 groups)
    assert [d.rows_per_tile for d in arr] == [32 * 14, 32 * 3, 32 * 4, 32 * 1]
    # the plan's variant is the largest tile's dynamic LDS: x (two copies for an
    # odd group count) and eight fp32 slots per row
    lds = [(2 * g if g % 2 else g) * 256 + r * 32
           for g, r in [(7, 448), (38, 96), (28, 128), (148, 32)]]
    assert plan_variant(arr) == max(lds)
    # other codings keep x in registers: K5 (16 weights per chunk), 896 columns
    # = 56 chunks -> 64 lanes x 1 pass
    arr = _descs(2, [(896, 896)])
    assert _prepare(arr)[0] == tkq.OK and _shape(arr[0]) == (64, 1, 1)


def plan_variant(arr):
    return _prepare(arr)[1].variant


def test_prepare_sweep_counts():
    shapes = [(n, k) for _, n, k in inputs.sweep_shapes("qwen2.5-0.5b")]
    arr = _descs(1, shapes)
    st, plan = _prepare(arr)
    assert st == tkq.OK and plan.count == 169 and plan.tiles > 1024


def test_prepare_validation():
    arr = _descs(1, [(8, 128), (8, 256)])
    arr[1].fmt = 2
    assert _prepare(arr)[0] == tkq.EFORMAT
    arr = _descs(99, [(8, 128)])
    assert _prepare(arr)[0] == tkq.EFORMAT
    arr = _descs(1, [(8, 200)])
    assert _prepare(arr)[0] == tkq.ESHAPE
    arr = _descs(1, [(8, 96)])                # int4 g128 needs K % 128
    assert _prepare(arr)[0] == tkq.ESHAPE
    arr = _descs(5, [(8, 96), (3, 32)])       # hier-g32 needs only K % 32
    assert _prepare(arr)[0] == tkq.OK
    arr = _descs(5, [(8, 112)])
    assert _prepare(arr)[0] == tkq.ESHAPE
    arr = _descs(5, [(8, 65536)])
    assert _prepare(arr)[0] == tkq.ESHAPE
    arr = _descs(1, [(8, 65536)])             # beyond the int4 GEMV's K
    assert _prepare(arr)[0] == tkq.ESHAPE
    arr = _descs(1, [(0, 128)])
    assert _prepare(arr)[0] == tkq.EINVAL
    arr = _descs(1, [(8, 128)])
    arr[0].meta = None
    assert _prepare(arr)[0] == tkq.EINVAL
    arr = _descs(4, [(8, 128)])
    arr[0].meta = None                        # binary needs no metadata
    assert _prepare(arr)[0] == tkq.OK
    arr = _descs(1, [(8, 128)])
    arr[0].x = A + 2
    assert _prepare(arr)[0] == tkq.EALIGN
    plan = tkq.GemvPlan()
    assert tkq.lib().tkq_gemv_prepare(arr, 0, ctypes.byref(plan)) == tkq.EINVAL


def test_gemv_rejects_unprepared_plan():
    plan = tkq.GemvPlan()
    plan.fmt, plan.count, plan.tiles = 1, 1, 1
    assert tkq.lib().tkq_gemv(ctypes.byref(plan), A, None) == tkq.EPLAN
    arr = _descs(1, [(8, 128)])
    st, plan = _prepare(arr)
    assert tkq.lib().tkq_gemv(ctypes.byref(plan), None, None) == tkq.EINVAL
    assert tkq.lib().tkq_gemv(ctypes.byref(plan), A + 8, None) == tkq.EALIGN


def test_gemv_argmax_validation():
    f = tkq.lib().tkq_gemv_argmax
    plan = tkq.GemvPlan()
    plan.fmt, plan.count, plan.tiles = 1, 1, 1
    assert f(ctypes.byref(plan), A, 0, A, A, 1 << 20, None) == tkq.EPLAN
    arr = _descs(1, [(8, 128), (16, 256)])
    st, plan = _prepare(arr)
    assert st == tkq.OK
    sb = 8 * plan.tiles
    assert f(ctypes.byref(plan), A, -1, A, A, sb, None) == tkq.EINVAL
    assert f(ctypes.byref(plan), A, 2, A, A, sb, None) == tkq.EINVAL
    assert f(ctypes.byref(plan), A, 1, None, A, sb, None) == tkq.EINVAL
    assert f(ctypes.byref(plan), A, 1, A, None, sb, None) == tkq.EINVAL
    assert f(ctypes.byref(plan), A, 1, A, A, sb - 8, None) == tkq.EINVAL
    assert f(ctypes.byref(plan), A, 1, A + 2, A, sb, None) == tkq.EALIGN
    assert f(ctypes.byref(plan), A, 1, A, A + 8, sb, None) == tkq.EALIGN
    assert f(ctypes.byref(plan), A + 8, 1, A, A, sb, None) == tkq.EALIGN


def test_gemv_argmax_static_validation():
    """The allocation-free greedy entry point rejects every bad argument on
    the host, before any HIP call, including plans with more row tiles than
    its fixed slot array holds."""
    f = tkq.lib().tkq_gemv_argmax_static
    plan = tkq.GemvPlan()
    plan.fmt, plan.count, plan.tiles = 1, 1, 1
    assert f(ctypes.byref(plan), A, 0, A, None) == tkq.EPLAN
    arr = _descs(1, [(8, 128), (16, 256)])
    st, plan = _prepare(arr)
    assert st == tkq.OK
    assert f(ctypes.byref(plan), A, -1, A, None) == tkq.EINVAL
    assert f(ctypes.byref(plan), A, 2, A, None) == tkq.EINVAL
    assert f(ctypes.byref(plan), A, 1, None, None) == tkq.EINVAL
    assert f(ctypes.byref(plan), A, 1, A + 2, None) == tkq.EALIGN
    assert f(ctypes.byref(plan), A + 8, 1, A, None) == tkq.EALIGN
    big = _descs(1, [(1, 128)] * 70000)             # one row tile each
    st, bplan = _prepare(big)
    assert st == tkq.OK and bplan.tiles > 65536
    assert f(ctypes.byref(bplan), A, 0, A, None) == tkq.ESHAPE


def test_gemm_small_prepare():
    f = tkq.lib().tkq_gemm_small_prepare
    arr = _descs(1, [(1, 128), (64, 896), (65, 896), (151936, 896)])
    plan = tkq.GemvPlan()
    assert f(arr, 4, 16, ctypes.byref(plan)) == tkq.OK
    rows = arr[0].rows_per_tile                    # one workgroup per tile of rows
    assert rows % 64 == 0 and all(d.rows_per_tile == rows for d in arr)
    tiles = [-(-n // rows) for n in (1, 64, 65, 151936)]
    assert [d.work0 for d in arr] == [0, tiles[0], sum(tiles[:2]), sum(tiles[:3])]
    assert plan.tiles == sum(tiles) and plan.variant == 16
    assert f(arr, 4, 17, ctypes.byref(plan)) == tkq.ESHAPE
    assert f(arr, 4, 0, ctypes.byref(plan)) == tkq.EINVAL
    bad = _descs(2, [(8, 128)])
    assert f(bad, 1, 4, ctypes.byref(plan)) == tkq.EFORMAT
    hier = _descs(5, [(8, 128), (65, 896)])       # int4-hier-g32 is taken too, one coding per call
    assert f(hier, 2, 4, ctypes.byref(plan)) == tkq.OK and plan.fmt == 5
    hier[1].fmt = 1
    assert f(hier, 2, 4, ctypes.byref(plan)) == tkq.EFORMAT
    assert f(_descs(5, [(8, 96)]), 1, 4, ctypes.byref(plan)) == tkq.ESHAPE   # K % 128 for both codings
    bad = _descs(1, [(8, 96)])
    assert f(bad, 1, 4, ctypes.byref(plan)) == tkq.ESHAPE
    # plans are not interchangeable between the batch-1 and multi-token entry points
    g = tkq.lib().tkq_gemm_small
    st, p1 = _prepare(_descs(1, [(8, 128)]))
    assert g(ctypes.byref(p1), A, None) == tkq.EPLAN
    assert f(arr, 4, 3, ctypes.byref(plan)) == tkq.OK
    assert tkq.lib().tkq_gemv(ctypes.byref(plan), A, None) == tkq.EPLAN
    assert g(ctypes.byref(plan), A + 8, None) == tkq.EALIGN


def test_kv_validation():
    L = tkq.lib()
    assert L.tkq_kv_cache_bytes(1, 32, 4096) == 32 * 32 * 17408
    assert L.tkq_kv_cache_bytes(1, 32, 100) == -1
    # arrival counters (4 bytes per sequence and head, to 16 bytes) + partials
    assert L.tkq_kv_decode_workspace_bytes(1, 32, 32, 4096) == 128 + 32 * 32 * 130 * 4
    assert L.tkq_kv_decode_workspace_bytes(1, 28, 4, 128) == 112 + 28 * 4 * 130 * 4   # 7 per KV head
    assert L.tkq_kv_decode_workspace_bytes(3, 1, 1, 128) == 16 + 3 * 4 * 130 * 4
    assert L.tkq_kv_decode_workspace_bytes(1, 8, 3, 128) == -1      # H % Hk != 0
    pk = L.tkq_kv_pack
    assert pk(None, A, 1, 128, 1, 128, A, None) == tkq.EINVAL
    assert pk(A, A, 1, 128, 1, 64, A, None) == tkq.ESHAPE             # D must be 128
    assert pk(A, A, 1, 200, 1, 128, A, None) == tkq.ESHAPE            # whole pages
    assert pk(A, A, 1, 128, 1, 128, A + 4, None) == tkq.EALIGN
    dec = L.tkq_kv_decode
    ws = L.tkq_kv_decode_workspace_bytes(1, 4, 2, 256)
    assert dec(A, A, 1, 4, 2, 256, 128, 0.1, A, A, ws - 4, None) == tkq.EINVAL
    assert dec(A, A, 1, 4, 2, 256, 128, 0.0, A, A, ws, None) == tkq.EINVAL
    assert dec(A, A, 1, 4, 2, 256, 128, float("nan"), A, A, ws, None) == tkq.EINVAL
    assert dec(A, A, 1, 4, 3, 256, 128, 0.1, A, A, ws, None) == tkq.ESHAPE
    assert dec(A, None, 1, 4, 2, 256, 128, 0.1, A, A, ws, None) == tkq.EINVAL
    assert dec(A + 2, A, 1, 4, 2, 256, 128, 0.1, A, A, ws, None) == tkq.EALIGN
    # per-sequence lengths: a null or misaligned length array is refused
    pv, dv = L.tkq_kv_pack_varlen, L.tkq_kv_decode_varlen
    assert pv(A, A, None, 1, 128, 1, 128, A, None) == tkq.EINVAL
    assert pv(A, A, A + 2, 1, 128, 1, 128, A, None) == tkq.EALIGN
    assert pv(A, A, A, 1, 200, 1, 128, A, None) == tkq.ESHAPE
    assert dv(A, A, None, 1, 4, 2, 256, 128, 0.1, A, A, ws, None) == tkq.EINVAL
    assert dv(A, A, A + 2, 1, 4, 2, 256, 128, 0.1, A, A, ws, None) == tkq.EALIGN
    assert dv(A, A, A, 1, 4, 2, 256, 128, 0.1, A, A, ws - 4, None) == tkq.EINVAL


def test_prefill_validation():
    f = tkq.lib().tkq_gemm_prefill
    assert f(2, 64, 128, 128, A, A, A, A, None, 0, None) == tkq.EFORMAT
    assert f(5, 64, 128, 128, A, A, A, A, None, 0, None) == tkq.EFORMAT
    assert f(1, 0, 128, 128, A, A, A, A, None, 0, None) == tkq.EINVAL
    assert f(1, 64, 128, 100, A, A, A, A, None, 0, None) == tkq.ESHAPE
    assert f(1, 64, 128, 128, None, A, A, A, None, 0, None) == tkq.EINVAL
    assert f(1, 64, 128, 128, A, A, A + 2, A, None, 0, None) == tkq.EALIGN
    assert f(1, 64, 128, 128, A, A, A, A, A, -4, None) == tkq.EINVAL
    assert f(1, 64, 128, 128, A, A, A, A, A, 0, None) == tkq.EINVAL
    assert f(1, 64, 128, 128, A, A, A, A, A + 4, 1 << 20, None) == tkq.EALIGN


def test_read_probe_validation():
    f = tkq.lib().tkq_read_probe
    assert f(None, 64, A, None) == tkq.EINVAL
    assert f(A, 8, A, None) == tkq.EINVAL
    assert f(A, 24, A, None) == tkq.ESHAPE
    assert f(A + 4, 64, A, None) == tkq.EALIGN


def test_head_rescore_validation():
    """Greedy selection with head rescore: every bad argument is refused on the
    host, including k beyond the candidate collection's capacity."""
    f = tkq.lib().tkq_head_rescore
    n, K = 151936, 896
    assert f(None, n, A, A, K, 64, A, None, None, None) == tkq.EINVAL
    assert f(A, n, None, A, K, 64, A, None, None, None) == tkq.EINVAL
    assert f(A, n, A, None, K, 64, A, None, None, None) == tkq.EINVAL
    assert f(A, n, A, A, K, 64, None, None, None, None) == tkq.EINVAL
    assert f(A, 0, A, A, K, 1, A, None, None, None) == tkq.EINVAL
    assert f(A, n, A, A, 0, 1, A, None, None, None) == tkq.EINVAL
    assert f(A, n, A, A, K, 0, A, None, None, None) == tkq.EINVAL
    assert f(A, 5, A, A, K, 6, A, None, None, None) == tkq.EINVAL       # k > n
    assert f(A, n, A, A, 900, 8, A, None, None, None) == tkq.ESHAPE     # K % 8
    assert f(A, n, A, A, (1 << 20) + 8, 8, A, None, None, None) == tkq.ESHAPE
    assert f(A, 1 << 31, A, A, K, 8, A, None, None, None) == tkq.ESHAPE
    assert f(A, 5000, A, A, K, 1025, A, None, None, None) == tkq.ESHAPE  # k > TKQ_RESCORE_MAX_K
    # capacity: k * 8 * ceil(ceil(n / 8) / 1024) <= 16384
    assert f(A, n, A, A, K, 108, A, None, None, None) == tkq.ESHAPE     # 108 * 152 > 16384
    assert f(A, 262145, A, A, K, 64, A, None, None, None) == tkq.ESHAPE
    assert f(A + 2, n, A, A, K, 8, A, None, None, None) == tkq.EALIGN
    assert f(A, n, A + 8, A, K, 8, A, None, None, None) == tkq.EALIGN
    assert f(A, n, A, A + 4, K, 8, A, None, None, None) == tkq.EALIGN
    assert f(A, n, A, A, K, 8, A + 2, None, None, None) == tkq.EALIGN
    assert f(A, n, A, A, K, 8, A, A + 1, None, None) == tkq.EALIGN
    assert f(A, n, A, A, K, 8, A, None, A + 2, None) == tkq.EALIGN


def test_gemv_argmax_rescore_validation():
    """The fused GEMV + head rescore entry point refuses every bad argument on
    the host (plan, target, coding, sizes, capacity, alignment)."""
    f = tkq.lib().tkq_gemv_argmax_rescore
    plan = tkq.GemvPlan()
    plan.fmt, plan.count, plan.tiles = 1, 1, 1
    assert f(ctypes.byref(plan), A, 0, 128, 128, A, 4, A, None, None, A, 1 << 20, None) == tkq.EPLAN
    arr = _descs(1, [(8, 128), (400, 256)])
    st, plan = _prepare(arr)
    assert st == tkq.OK
    sb = 8 * plan.tiles
    ok = (A, 1, 400, 256, A, 4, A, None, None, A, sb, None)

    def call(**kw):
        names = ["descs", "target", "N", "K", "head", "k", "token", "cand", "cl", "scratch", "sb", "stream"]
        args = dict(zip(names, ok))
        args.update(kw)
        return f(ctypes.byref(plan), *[args[n] for n in names])
    assert call(target=-1) == tkq.EINVAL
    assert call(target=2) == tkq.EINVAL
    assert call(head=None) == tkq.EINVAL
    assert call(token=None) == tkq.EINVAL
    assert call(scratch=None) == tkq.EINVAL
    assert call(sb=sb - 8) == tkq.EINVAL
    assert call(N=0) == tkq.EINVAL
    assert call(K=0) == tkq.EINVAL
    assert call(k=0) == tkq.EINVAL
    assert call(k=401) == tkq.EINVAL
    assert call(K=260) == tkq.ESHAPE
    assert call(N=151936, k=108) == tkq.ESHAPE
    assert call(N=5000, k=1025) == tkq.ESHAPE
    assert call(head=A + 8) == tkq.EALIGN
    assert call(scratch=A + 8) == tkq.EALIGN
    assert call(token=A + 2) == tkq.EALIGN
    assert call(cand=A + 1) == tkq.EALIGN
    assert call(cl=A + 2) == tkq.EALIGN
    assert call(descs=A + 8) == tkq.EALIGN
    bin_arr = _descs(4, [(8, 128)])
    st, bplan = _prepare(bin_arr)
    assert st == tkq.OK
    assert f(ctypes.byref(bplan), A, 0, 8, 128, A, 4, A, None, None, A, 1 << 20, None) == tkq.EFORMAT

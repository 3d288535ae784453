"""Shared helpers of the GPU parity tests: device checks, dtype views, and the
oracle-side packing of a coding (test infrastructure)."""

import os

import numpy as np
import pytest

from oracle import pack as opack
from oracle import quant as oquant
from oracle import ref as oref

FMTS = ("int4", "k5", "tern", "bin", "hier", "int2", "int3")


def gpu_or_skip():
    """Skip when there is no GPU; fail loudly when the GPU is there but the
    HIP library is not built (never fall back to anything else)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gemm_tkq_gemv_amd import tkq
    if not os.path.exists(tkq.LIB_PATH):
        raise RuntimeError("GPU present but libtkq.so is not built")
    tkq.lib()
    return torch


def u32(t):
    """int32 device tensor of packed words -> numpy uint32 (same bits)."""
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def f16bits(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint16)


def oracle_pack(fmt, W):
    """Oracle codes and metadata in the library's storage layout (numpy)."""
    if fmt == "int4":
        q, s, z = oquant.quantize_int4_g128(W)
        return opack.pack_int4(q), opack.pack_int4_meta(s, z)
    if fmt == "k5":
        c, s = oquant.quantize_k5(W)
        return c, s
    if fmt == "tern":
        c, s = oquant.quantize_tern_g128(W)
        return opack.pack_tern(c), s
    if fmt == "bin":
        return opack.pack_bits(oquant.sign_bits(W)), None
    if fmt == "int2":
        q, s, z = oquant.quantize_int2_g128(W)
        return opack.pack_int2(q), opack.pack_int4_meta(s, z)
    if fmt == "int3":
        q, s, z = oquant.quantize_int3_g128(W)
        return opack.pack_int3(q), opack.pack_int4_meta(s, z)
    if fmt == "hier":
        q, sc, mi, d16, dmin16 = oquant.quantize_int4_hier_g32(W)
        return opack.pack_int4(q), opack.pack_hier_meta(sc, mi, d16, dmin16)
    raise ValueError(fmt)


def oracle_wdeq(fmt, codes, meta, K):
    """fp64 dequantized weights from stored (numpy) codes and metadata."""
    if fmt == "int4":
        return oref.dequant_int4(codes, meta, K)
    if fmt == "k5":
        return oref.dequant_k5(codes, meta)
    if fmt == "tern":
        return oref.dequant_tern(codes, meta, K)
    if fmt == "hier":
        return oref.dequant_int4_hier(codes, meta, codes.shape[0], K)
    if fmt == "int2":
        return oref.dequant_int2(codes, meta, K)
    if fmt == "int3":
        return oref.dequant_int3(codes, meta, K)
    raise ValueError(fmt)


def device_codes_np(fmt, codes, meta):
    """Device packed tensors -> numpy arrays in the oracle's dtypes."""
    if fmt in ("int4", "int2", "int3"):
        return u32(codes), u32(meta)
    if fmt == "k5":
        return codes.cpu().numpy(), meta.cpu().numpy()
    if fmt == "tern":
        return u32(codes), meta.cpu().numpy()
    if fmt == "hier":
        return u32(codes), meta.cpu().numpy()
    return u32(codes), None


def hier_meta_rows(meta, N, K, rows):
    """The metadata block of selected rows of an int4-hier-g32 matrix (from
    the full block as a numpy uint8 array), re-laid out for those rows."""
    sc, mi, d16, dmin16 = opack.unpack_hier_meta(meta, N, K)
    return opack.pack_hier_meta(sc[rows], mi[rows], d16[rows], dmin16[rows])


def device_rows_np(fmt, codes, meta, N, K, rows):
    """Packed codes and metadata of selected rows, as device_codes_np would
    give for a matrix of just those rows."""
    import torch
    rows = np.asarray(rows)
    # int3 codes are plane-major [3][N][K/32]: rows are the second index
    row_dim = 1 if fmt == "int3" else 0
    # checked on the host: an index past the end would fail on the device
    assert codes.shape[row_dim] == N and rows.min() >= 0 and rows.max() < N
    rt = torch.from_numpy(rows).to(codes.device)
    if fmt == "hier":
        return u32(codes[rt]), hier_meta_rows(meta.cpu().numpy(), N, K, rows)
    if fmt == "int3":
        return device_codes_np(fmt, codes[:, rt], meta[rt])
    return device_codes_np(fmt, codes[rt], None if meta is None else meta[rt])


def assert_codes_equal(fmt, got, want):
    gc, gm = got
    wc, wm = want
    assert np.array_equal(gc, wc), "%s codes differ at %s" % (fmt, np.argwhere(gc != wc)[:5])
    if wm is not None:
        a = np.asarray(gm).view(np.uint16) if np.asarray(gm).dtype == np.float16 else np.asarray(gm)
        b = np.asarray(wm).view(np.uint16) if np.asarray(wm).dtype == np.float16 else np.asarray(wm)
        assert np.array_equal(a, b), "%s metadata differ at %s" % (fmt, np.argwhere(a != b)[:5])


def check_gemv(y_gpu, w_deq, x, what=""):
    """Per-row bound |y - y_ref| <= 2e-3 * sum|w x| (fp64 oracle)."""
    y_ref = oref.gemv(w_deq, x.astype(np.float64))
    bound = oref.gemv_bound(w_deq, x.astype(np.float64))
    ok, worst = oref.check_within(np.asarray(y_gpu, np.float64), y_ref, bound)
    assert ok, "%s: worst |err|/bound = %g" % (what, worst)
    return worst


def tile_edge_rows(desc):
    """First and last row of every row tile of a prepared descriptor (large
    tiles of rows_per_tile rows at the top, small tiles of small_rows below;
    the last tile may overhang N)."""
    N, big, rpt, sr = desc.N, desc.big_tiles, desc.rows_per_tile, desc.small_rows
    starts = [t * rpt for t in range(big)]
    r = big * rpt
    while r < N:
        starts.append(r)
        r += sr
    edges = []
    for a, b in zip(starts, starts[1:] + [N]):
        edges += [a, min(b, N) - 1]
    return np.unique(np.asarray(edges, dtype=np.int64))

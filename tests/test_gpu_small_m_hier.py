"""GPU multi-token GEMV over int4-hier-g32 weights (tkq_gemm_small with the
two-level coding: Whetstone README, quantizer table, "group 32 with
hierarchical scale metadata", and "Prior art" on several tokens sharing a
weight read) against the fp64 oracle Y = X . W_deq^T.

Bound, entry-wise: 2e-3 * sum_k |X[m,k]| (|d sc q| + |dmin mi|).  The
kernel forms each weight in fp16 from the step d sc and the offset dmin mi
(each rounded once) with one fused multiply-add, so its error follows the
two terms, not their difference; the fp32 sum and the fp16 output rounding
fit in the rest of the factor.  The codes packed on the GPU are checked to
be the oracle's on every case.  Unit tokens pin the documented rounding
exactly: fp16(q * fp16(d sc) - fp16(dmin mi)), taken once."""

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
from helpers import assert_codes_equal, device_codes_np, gpu_or_skip, oracle_pack, oracle_wdeq
from oracle import pack as opack
from oracle import ref as oref

pytestmark = pytest.mark.gpu


def _items(torch, tkq, mats, M):
    items = []
    for W, X in mats:
        N, K = W.shape
        codes, meta = tkq.pack_int4_hier_g32(torch.from_numpy(W).cuda())
        Y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        items.append(dict(codes=codes, meta=meta, x=torch.from_numpy(X).cuda(), y=Y, N=N, K=K))
    return items


def _terms(oc, om, N, K):
    """|d sc q| + |dmin mi| per weight (fp64) from the oracle's packed form."""
    q = opack.unpack_int4(oc, K).astype(np.float64)
    sc, mi, d16, dmin16 = opack.unpack_hier_meta(om, N, K)
    step = np.repeat(d16.astype(np.float64)[:, None] * sc, 32, axis=1)
    off = np.repeat(dmin16.astype(np.float64)[:, None] * mi, 32, axis=1)
    return np.abs(step * q) + np.abs(off)


def _check(W, X, item, what):
    N, K = W.shape
    oc, om = oracle_pack("hier", W)
    assert_codes_equal("hier", device_codes_np("hier", item["codes"], item["meta"]), (oc, om))
    w_deq = oracle_wdeq("hier", oc, om, K)
    X64 = X.astype(np.float64)
    bound = oref.TOL * (np.abs(X64) @ _terms(oc, om, N, K).T)
    ok, worst = oref.check_within(item["y"].float().cpu().numpy(), oref.gemm(X64, w_deq), bound)
    assert ok, "%s: worst |err|/bound = %g" % (what, worst)
    return worst


def _X(seed, M, K):
    return np.stack([inputs.normal_vector((seed, m), K) for m in range(M)])


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 9, 12, 16])
def test_small_m_hier_each_m(M):
    """Both staging variants (1024 columns per round for M <= 8, 512 above),
    6 tiles with a ragged last one, K = 1152 ending mid-round."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K = 333, 1152
    W = inputs.normal_matrix((760, N, K), N, K)
    X = _X(761, M, K)
    items = _items(torch, tkq, [(W, X)], M)
    tkq.GemvBatch("hier", items, tokens=M).run()
    torch.cuda.synchronize()
    _check(W, X, items[0], "M=%d" % M)


@pytest.mark.parametrize("M", [2, 16])
def test_small_m_hier_grouped_shapes(M):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    shapes = [(1, 128), (64, 128), (65, 896), (896, 896), (128, 896), (4864, 896), (896, 4864),
              (300, 18944), (2049, 384), (7, 640)]
    mats = [(inputs.normal_matrix((770, i), n, k), _X((771, i), M, k)) for i, (n, k) in enumerate(shapes)]
    items = _items(torch, tkq, mats, M)
    batch = tkq.GemvBatch("hier", items, tokens=M)
    batch.run()
    torch.cuda.synchronize()
    first = [it["y"].clone() for it in items]
    worst = 0.0
    for (W, X), it in zip(mats, items):
        worst = max(worst, _check(W, X, it, "M=%d %s" % (M, W.shape)))
    for it in items:                       # a second launch is bit-identical
        it["y"].fill_(0)
    batch.run()
    torch.cuda.synchronize()
    for a, it in zip(first, items):
        assert torch.equal(a, it["y"])
    print("M=%d worst |err|/bound %.3g" % (M, worst))


def test_small_m_hier_unit_tokens_exact():
    """A token with a single 1 at column k returns that column's fp16 weight:
    q * S - O rounded once, with S = fp16(d sc) and O = fp16(dmin mi).  The
    products of fp16 numbers by 4-bit integers and their difference are
    exact in fp64, so one conversion to fp16 is the fused rounding."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K, M = 500, 896, 7
    cols = (0, 5, 31, 32, 127, 128, 895)
    W = inputs.normal_matrix((780, N, K), N, K)
    X = np.zeros((M, K), np.float16)
    for m, k in enumerate(cols):
        X[m, k] = 1
    items = _items(torch, tkq, [(W, X)], M)
    tkq.GemvBatch("hier", items, tokens=M).run()
    torch.cuda.synchronize()
    oc, om = oracle_pack("hier", W)
    q = opack.unpack_int4(oc, K).astype(np.float64)
    sc, mi, d16, dmin16 = opack.unpack_hier_meta(om, N, K)
    Y = items[0]["y"].cpu().numpy()
    for m, k in enumerate(cols):
        g = k // 32
        S = (d16.astype(np.float64) * sc[:, g]).astype(np.float16).astype(np.float64)
        O = (dmin16.astype(np.float64) * mi[:, g]).astype(np.float16).astype(np.float64)
        want = (q[:, k] * S - O).astype(np.float16)
        assert np.array_equal(Y[m].view(np.uint16), want.view(np.uint16)), k


def test_small_m_hier_zero_rows_and_tokens():
    """A zero row (its row pair is zero) and a zero token give zeros."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K, M = 130, 4864, 16
    W = inputs.normal_matrix((790, N, K), N, K)
    W[3] = 0.0
    X = _X(791, M, K)
    X[4] = 0
    items = _items(torch, tkq, [(W, X)], M)
    tkq.GemvBatch("hier", items, tokens=M).run()
    torch.cuda.synchronize()
    Y = items[0]["y"].float().cpu().numpy()
    assert np.all(np.isfinite(Y))
    assert np.all(Y[4] == 0) and np.all(Y[:, 3] == 0)
    _check(W, X, items[0], "zeros")


def test_small_m_hier_matches_gemv_bound():
    """Every token row lies within the same oracle bound as the batch-1
    int4-hier-g32 GEMV of that token (both paths, one packed matrix)."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K, M = 700, 2432, 4
    W = inputs.normal_matrix((800, N, K), N, K)
    X = _X(801, M, K)
    items = _items(torch, tkq, [(W, X)], M)
    tkq.GemvBatch("hier", items, tokens=M).run()
    ys = []
    for m in range(M):
        y = torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
        it = dict(items[0], x=items[0]["x"][m].contiguous(), y=y)
        tkq.GemvBatch("hier", [it]).run()
        ys.append(y)
    torch.cuda.synchronize()
    _check(W, X, items[0], "multi-token")
    oc, om = oracle_pack("hier", W)
    terms = _terms(oc, om, N, K)
    w_deq = oracle_wdeq("hier", oc, om, K)
    for m in range(M):
        x64 = X[m].astype(np.float64)
        ok, worst = oref.check_within(ys[m].float().cpu().numpy(), oref.gemv(w_deq, x64),
                                      oref.TOL * (terms @ np.abs(x64)))
        assert ok, "batch-1 token %d: %g" % (m, worst)


def test_small_m_hier_max_k():
    """K = 2^20 (the multi-token limit), 9 rows, 16 tokens."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K, M = 9, 1 << 20, 16
    W = inputs.normal_matrix((810, N, K), N, K)
    X = _X(811, M, K)
    items = _items(torch, tkq, [(W, X)], M)
    tkq.GemvBatch("hier", items, tokens=M).run()
    torch.cuda.synchronize()
    _check(W, X, items[0], "M=16 9x2^20")


@pytest.mark.parametrize("M", [3, 16])
def test_small_m_hier_large_activations(M):
    """Activations of 1e3..3e4 on all-zero weight columns, heavy-tailed
    weights with one outlier per 32-group: the two-term bound holds."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    from test_gpu_small_m import _outlier_tokens
    N, K = 200, 4864
    W, X = _outlier_tokens((820, M), N, K, M, 32)
    assert np.abs(X.astype(np.float32)).max() >= 1e3
    items = _items(torch, tkq, [(W, X)], M)
    tkq.GemvBatch("hier", items, tokens=M).run()
    torch.cuda.synchronize()
    _check(W, X, items[0], "outliers M=%d" % M)

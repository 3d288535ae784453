"""GPU multi-token GEMV (tkq_gemm_small, M = 1..16 tokens over int4 g128
weights) against the fp64 oracle Y = X . W_deq^T, entry-wise within
2e-3 * sum_k |x w|; codes packed on the GPU are the oracle's (checked in
test_gpu_pack).  Covers every M, ragged N (tiles of 64 rows), K not a
multiple of the 512-column staging round, grouped launches of mixed shapes,
the 0.5B sweep's shapes, and row-by-row agreement with the batch-1 GEMV."""

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
from helpers import gpu_or_skip, oracle_pack, oracle_wdeq
from oracle import ref as oref

pytestmark = pytest.mark.gpu


def _items(torch, tkq, mats, M):
    items = []
    for W, X in mats:
        N, K = W.shape
        codes, meta = tkq.pack_int4_g128(torch.from_numpy(W).cuda())
        Y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        items.append(dict(codes=codes, meta=meta, x=torch.from_numpy(X).cuda(), y=Y, N=N, K=K))
    return items


def _check(W, X, Y, what):
    oc, om = oracle_pack("int4", W)
    w_deq = oracle_wdeq("int4", oc, om, W.shape[1])
    X64 = X.astype(np.float64)
    ok, worst = oref.check_within(Y.float().cpu().numpy(), oref.gemm(X64, w_deq), oref.gemm_bound(X64, w_deq))
    assert ok, "%s: worst |err|/bound = %g" % (what, worst)
    return worst


def _X(seed, M, K):
    return np.stack([inputs.normal_vector((seed, m), K) for m in range(M)]) if M else None


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_small_m_every_m(M):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K = 333, 1152                      # 6 tiles (ragged), 2 staging rounds (512 + 512 + 128)
    W = inputs.normal_matrix((700, N, K), N, K)
    X = _X(701, M, K)
    items = _items(torch, tkq, [(W, X)], M)
    tkq.GemvBatch("int4", items, tokens=M).run()
    torch.cuda.synchronize()
    _check(W, X, items[0]["y"], "M=%d" % M)


@pytest.mark.parametrize("M", [2, 7, 16])
def test_small_m_grouped_shapes(M):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    shapes = [(1, 128), (64, 128), (65, 896), (896, 896), (128, 896), (4864, 896), (896, 4864),
              (300, 18944), (2049, 384)]
    mats = [(inputs.normal_matrix((710, i), n, k), _X((711, i), M, k)) for i, (n, k) in enumerate(shapes)]
    items = _items(torch, tkq, mats, M)
    batch = tkq.GemvBatch("int4", items, tokens=M)
    batch.run()
    torch.cuda.synchronize()
    first = [it["y"].clone() for it in items]
    worst = 0.0
    for (W, X), it in zip(mats, items):
        worst = max(worst, _check(W, X, it["y"], "M=%d %s" % (M, W.shape)))
    for it in items:                       # a second launch is bit-identical
        it["y"].fill_(0)
    batch.run()
    torch.cuda.synchronize()
    for a, it in zip(first, items):
        assert torch.equal(a, it["y"])
    print("M=%d worst |err|/bound %.3g" % (M, worst))


def test_small_m_rows_match_gemv_bound():
    """Each token's row of Y is a GEMV of the same weights: both paths are
    within the bound of the same oracle row, and unit tokens pick out
    fp16-rounded dequantized columns exactly."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K, M = 500, 896, 5
    W = inputs.normal_matrix((720, N, K), N, K)
    X = np.zeros((M, K), np.float16)
    for m, k in enumerate((0, 5, 127, 128, 895)):
        X[m, k] = 1
    items = _items(torch, tkq, [(W, X)], M)
    tkq.GemvBatch("int4", items, tokens=M).run()
    torch.cuda.synchronize()
    oc, om = oracle_pack("int4", W)
    w_deq = oracle_wdeq("int4", oc, om, K)
    Y = items[0]["y"].cpu().numpy()
    for m, k in enumerate((0, 5, 127, 128, 895)):
        want = w_deq[:, k].astype(np.float16)     # s*(q-z) rounded once, times 1, fp32 sum of zeros
        assert np.array_equal(Y[m].view(np.uint16), want.view(np.uint16)), k


def test_small_m_zero_tokens_are_zero_and_finite():
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K, M = 130, 4864, 16
    W = inputs.normal_matrix((730, N, K), N, K)
    W[3] = 0.0
    X = _X(731, M, K)
    X[4] = 0
    items = _items(torch, tkq, [(W, X)], M)
    tkq.GemvBatch("int4", items, tokens=M).run()
    torch.cuda.synchronize()
    Y = items[0]["y"].float().cpu().numpy()
    assert np.all(np.isfinite(Y))
    assert np.all(Y[4] == 0) and np.all(Y[:, 3] == 0)
    _check(W, X, items[0]["y"], "zeros")


def test_small_m_max_k():
    """The longest rows the multi-token path takes (K = 2^20, the header's
    limit): 9 rows, 16 tokens, 1024 staging rounds; K one group further is
    refused."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K, M = 9, 1 << 20, 16
    W = inputs.normal_matrix((740, N, K), N, K)
    X = _X(741, M, K)
    items = _items(torch, tkq, [(W, X)], M)
    tkq.GemvBatch("int4", items, tokens=M).run()
    torch.cuda.synchronize()
    _check(W, X, items[0]["y"], "M=16 9x2^20")
    with pytest.raises(tkq.TkqError):
        tkq.GemvBatch("int4", [dict(items[0], K=K + 128)], tokens=M)


def _outlier_tokens(seed, N, K, M, group):
    """W and M tokens that share the outlier recipe of the batch-1 tests:
    heavy-tailed weights, one outlier weight per group, and two channels per
    group of 1e3..3e4 on all-zero weight columns (signs drawn per token)."""
    W, x0 = inputs.outlier_case(seed, N, K, group)
    big = np.abs(x0.astype(np.float32)) >= 1e3
    r = np.random.default_rng((*seed, 1))
    X = r.standard_normal((M, K)).astype(np.float32)
    X[:, big] = x0[big].astype(np.float32) * r.choice([-1.0, 1.0], (M, int(big.sum())))
    return W, X.astype(np.float16)


@pytest.mark.parametrize("M", [3, 16])
def test_small_m_large_activations(M):
    """Activations of 1e3..3e4 on weights at their zero point: the entry-wise
    bound holds (the weights are exact fp16 s (q - z) and the products exact
    in fp32, so the error follows |x w|, not the activations' size)."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K = 200, 4864
    W, X = _outlier_tokens((750, M), N, K, M, 128)
    assert np.abs(X.astype(np.float32)).max() >= 1e3
    items = _items(torch, tkq, [(W, X)], M)
    tkq.GemvBatch("int4", items, tokens=M).run()
    torch.cuda.synchronize()
    _check(W, X, items[0]["y"], "outliers M=%d" % M)

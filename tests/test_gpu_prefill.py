"""GPU prefill GEMM (int4 g128 weights, fp16 MFMA) against the fp64 oracle:
entry-wise bound over the k-sum, ragged shapes, the 7B-shaped M = 512
gate/up/down GEMMs in full, and consistency with the GEMV row by row."""

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
from helpers import gpu_or_skip, oracle_pack, oracle_wdeq
from oracle import ref as oref

pytestmark = pytest.mark.gpu


def _run(torch, tkq, W, X, split=False):
    codes, meta = tkq.pack_int4_g128(torch.from_numpy(W).cuda())
    ws = None
    if split:   # room for 8 partial products: lets the library split K
        ws = torch.full((8 * X.shape[0] * W.shape[0],), float("nan"), dtype=torch.float32, device="cuda")
    Y = tkq.gemm_prefill(codes, meta, torch.from_numpy(X).cuda(), W.shape[0], workspace=ws)
    torch.cuda.synchronize()
    return codes, meta, Y


def _check(Y, X, w_deq, what):
    Yr = oref.gemm(X, w_deq)
    ok, worst = oref.check_within(Y.float().cpu().numpy(), Yr, oref.gemm_bound(X, w_deq))
    assert ok, "%s: worst |err|/bound = %g" % (what, worst)
    return worst


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (64, 128, 256), (65, 200, 384),
                                   (130, 333, 896), (512, 256, 1024), (257, 129, 4864),
                                   (512, 96, 8192), (33, 1000, 640),
                                   (200, 33000, 256)])   # > one round of tiles: tail split with a workspace
def test_prefill_ragged(M, N, K, split):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    W = inputs.normal_matrix((500, M, N, K), N, K)
    X = np.random.default_rng((501, M, K)).standard_normal((M, K), dtype=np.float32).astype(np.float16)
    _, _, Y = _run(torch, tkq, W, X, split)
    oc, om = oracle_pack("int4", W)
    _check(Y, X, oracle_wdeq("int4", oc, om, K), "%dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("name,split", [("gate", False), ("gate", True), ("up", True), ("down", True)])
def test_prefill_7b_mlp_full(name, split):
    """With a workspace, gate/up (592 tiles: two rounds per XCD, the second
    partial) take the tail split, down (224 tiles) the split-K path."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    W = inputs.prefill_W(name)
    N, K = W.shape
    X = inputs.prefill_X(K)
    codes, meta, Y = _run(torch, tkq, W, X, split=split)
    oc, om = oracle_pack("int4", W)
    worst = _check(Y, X, oracle_wdeq("int4", oc, om, K), name)
    print("prefill %s worst |err|/bound %.3g" % (name, worst))
    # row m of the GEMM equals the GEMV of X[m] within the same bound
    xm = torch.from_numpy(X[7]).cuda()
    y = tkq.gemv("int4", codes, meta, xm, N, K)
    torch.cuda.synchronize()
    diff = np.abs(y.float().cpu().numpy().astype(np.float64) - Y[7].float().cpu().numpy())
    w_deq = oracle_wdeq("int4", oc, om, K)
    assert np.all(diff <= 2 * oref.gemv_bound(w_deq, X[7].astype(np.float64)))


@pytest.mark.parametrize("split", [False, True])
def test_prefill_max_k(split):
    """K = 2^20 (the header's limit): 16,384 K steps per tile without a
    workspace, split over K with one."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    M, N, K = 65, 9, 1 << 20
    W = inputs.normal_matrix((510, N, K), N, K)
    X = np.random.default_rng((511, M, K)).standard_normal((M, K), dtype=np.float32).astype(np.float16)
    _, _, Y = _run(torch, tkq, W, X, split)
    oc, om = oracle_pack("int4", W)
    _check(Y, X, oracle_wdeq("int4", oc, om, K), "%dx%dx%d" % (M, N, K))

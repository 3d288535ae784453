"""GPU grouped GEMV with fused greedy selection (tkq_gemv_argmax) against the
oracle.  Several tokens can be correct only when logits tie within the GEMV
tolerance, so the check is: (1) the token is exactly the first-index argmax
of the GPU's own stored outputs (oracle.ref.greedy_token), (2) the outputs
are within the per-row bound of the fp64 oracle, and (3) the chosen row's
exact logit is within the two rows' bounds of the exact maximum.  The
scratch buffer starts with garbage: the result may not depend on it."""

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
from helpers import check_gemv, gpu_or_skip, oracle_pack, oracle_wdeq
from oracle import ref as oref

pytestmark = pytest.mark.gpu


def _pack(tkq, fmt, Wd):
    return {"int4": tkq.pack_int4_g128, "k5": tkq.pack_k5, "tern": tkq.pack_tern_g128,
            "hier": tkq.pack_int4_hier_g32, "int2": tkq.pack_int2_g128, "int3": tkq.pack_int3_g128}[fmt](Wd)


def _run(torch, tkq, fmt, mats, target, calls=1):
    items = []
    for W, x in mats:
        N, K = W.shape
        codes, meta = _pack(tkq, fmt, torch.from_numpy(W).cuda())
        y = torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
        items.append(dict(codes=codes, meta=meta, x=torch.from_numpy(x).cuda(), y=y, N=N, K=K))
    batch = tkq.GemvBatch(fmt, items)
    token = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    scratch = batch.greedy_scratch()
    toks = []
    for i in range(calls):
        token.fill_(-1)
        scratch.random_(0, 2 ** 62, generator=torch.Generator("cuda").manual_seed(i))
        batch.run_argmax(target, token, scratch)
        torch.cuda.synchronize()
        toks.append(int(token.item()))
    return items, toks


def _check_choice(fmt, W, x, y_gpu, tok):
    yf = y_gpu.float().cpu().numpy()
    assert tok == oref.greedy_token(y_gpu.cpu().numpy()), "token is not the first argmax of the stored y"
    oc, om = oracle_pack(fmt, W)
    w_deq = oracle_wdeq(fmt, oc, om, W.shape[1])
    check_gemv(yf, w_deq, x, "greedy %s" % fmt)
    y_ref = oref.gemv(w_deq, x.astype(np.float64))
    bound = oref.gemv_bound(w_deq, x.astype(np.float64))
    best = int(np.argmax(y_ref))
    assert y_ref[tok] >= y_ref[best] - bound[tok] - bound[best]


@pytest.mark.parametrize("fmt", ["int4", "hier"])
def test_greedy_lm_head_shape(fmt):
    """The 0.5B output projection (151936 x 896) alone, three calls."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    W, x = inputs.sweep_matrix("qwen2.5-0.5b", 168, 151936, 896)
    items, toks = _run(torch, tkq, fmt, [(W, x)], 0, calls=3)
    assert toks[0] == toks[1] == toks[2]
    _check_choice(fmt, W, x, items[0]["y"], toks[0])


@pytest.mark.parametrize("fmt", ["int4", "k5", "tern", "int2", "int3"])
def test_greedy_target_inside_group(fmt):
    """A grouped launch of mixed shapes; the target is the first, a middle and
    the last descriptor in turn; other matrices' outputs are unaffected."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    shapes = [(896, 896), (128, 896), (4864, 896), (896, 4864), (20000, 896)]
    mats = [(inputs.normal_matrix((600, i), n, k), inputs.normal_vector((601, i), k))
            for i, (n, k) in enumerate(shapes)]
    for target in (0, 3, 4):
        items, toks = _run(torch, tkq, fmt, mats, target)
        W, x = mats[target]
        _check_choice(fmt, W, x, items[target]["y"], toks[0])
        for (Wi, xi), it in zip(mats, items):                     # every GEMV still right
            oc, om = oracle_pack(fmt, Wi)
            check_gemv(it["y"].float().cpu().numpy(), oracle_wdeq(fmt, oc, om, Wi.shape[1]), xi, fmt)


def test_greedy_ties_and_negatives():
    """Equal maxima pick the smallest row; an all-negative output vector."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K = 40000, 896
    W = inputs.normal_matrix((610, N, K), N, K)
    x = inputs.normal_vector(611, K)
    hot = (x.astype(np.float32) * np.float32(0.05)).astype(np.float32)
    for r in (29999, 7, 12345):           # three identical rows -> identical outputs
        W[r] = hot
    items, toks = _run(torch, tkq, "int4", [(W, x)], 0)
    assert toks[0] == 7
    _check_choice("int4", W, x, items[0]["y"], toks[0])
    Wn = -np.abs(W) - np.float32(0.01)
    xp = np.abs(x).astype(np.float16)
    items, toks = _run(torch, tkq, "int4", [(Wn, xp)], 0)
    assert float(items[0]["y"].float().max()) < 0
    _check_choice("int4", Wn, xp, items[0]["y"], toks[0])


def test_greedy_k_slices():
    """K = 18944 runs with four k-slices per row (outputs finished after the
    LDS reduction): the selection covers that path too."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K = 3000, 18944
    W = inputs.normal_matrix((620, N, K), N, K)
    x = inputs.normal_vector(621, K)
    items, toks = _run(torch, tkq, "int4", [(W, x)], 0, calls=2)
    assert toks[0] == toks[1]
    _check_choice("int4", W, x, items[0]["y"], toks[0])


def test_greedy_binary():
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K = 4864, 896
    W, x = inputs.binary_case(N, K)
    bits = tkq.pack_bin(torch.from_numpy(W).cuda())
    xb = tkq.pack_bin(torch.from_numpy(x).cuda())
    y = torch.full((N,), -7, dtype=torch.int32, device="cuda")
    batch = tkq.GemvBatch("bin", [dict(codes=bits, meta=None, x=xb, y=y, N=N, K=K)])
    token = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    batch.run_argmax(0, token, batch.greedy_scratch().fill_(-1))
    torch.cuda.synchronize()
    want = oref.bin_dot(W, x)
    assert np.array_equal(y.cpu().numpy(), want)
    assert int(token.item()) == oref.greedy_token(want)

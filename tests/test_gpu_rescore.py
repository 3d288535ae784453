"""GPU greedy selection with head rescore (tkq_head_rescore) against the
oracle (oracle.rescore).

The candidate rows are index work on the GPU's own stored logits, so they
must equal the oracle's candidates exactly, in order.  The recomputed logits
are fp32 sums of exact fp16 products: each must lie within the oracle's
summation bound of its exact (fp64) value.  The token must be exactly the
selection rule applied to the GPU's recomputed logits, and its exact logit
must be within the two rows' bounds of the best exact candidate logit."""

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
from helpers import gpu_or_skip
from oracle import ref as oref
from oracle import rescore as ores

pytestmark = pytest.mark.gpu


def _order_key(v, i):
    return (0, 0.0, i) if np.isnan(v) else (1, -float(v), i)


def _rescore(torch, tkq, logits16, head16, x16, k, calls=1):
    """Run tkq_head_rescore on numpy fp16 inputs; returns (token, cand, cand_logits)."""
    y = torch.from_numpy(np.ascontiguousarray(logits16)).cuda()
    h = torch.from_numpy(np.ascontiguousarray(head16)).cuda()
    x = torch.from_numpy(np.ascontiguousarray(x16)).cuda()
    return _rescore_dev(torch, tkq, y, h, x, k, calls)


def _rescore_dev(torch, tkq, y, h, x, k, calls=1):
    outs = []
    for i in range(calls):
        token = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        cand = torch.full((k,), -7, dtype=torch.int32, device="cuda")
        cl = torch.full((k,), float("nan"), dtype=torch.float32, device="cuda")
        tkq.head_rescore(y, h, x, k, token=token, cand=cand, cand_logits=cl)
        torch.cuda.synchronize()
        outs.append((int(token.item()), cand.cpu().numpy(), cl.cpu().numpy()))
    for o in outs[1:]:
        assert o[0] == outs[0][0] and np.array_equal(o[1], outs[0][1])
        assert np.array_equal(o[2].view(np.uint32), outs[0][2].view(np.uint32))
    return outs[0]


def _check(logits16, head_rows, x16, k, tok, cand, cl, what):
    """head_rows(rows) -> fp16 numpy rows of the head (so that huge heads
    need not be copied back whole)."""
    want = ores.candidates(logits16, k)
    assert np.array_equal(cand, want), "%s: candidate rows differ from the oracle's" % what
    H = head_rows(want)
    exact = ores.recompute(H, x16, np.arange(len(want)))
    bound = ores.recompute_bound(H, x16, np.arange(len(want)))
    fin = np.isfinite(exact)
    assert np.array_equal(np.isnan(cl), np.isnan(exact)), "%s: NaN pattern" % what
    assert np.all(cl[~fin & ~np.isnan(exact)] == exact[~fin & ~np.isnan(exact)]), "%s: infinities" % what
    err = np.abs(cl[fin].astype(np.float64) - exact[fin])
    assert np.all(err <= bound[fin]), "%s: recomputed logit off by %g (bound %g)" % (
        what, float(np.max(err - bound[fin])), 0.0)
    # the selection step, exactly, on the GPU's own recomputed logits
    j = min(range(k), key=lambda i: _order_key(cl[i], int(cand[i])))
    assert tok == int(cand[j]), "%s: token is not the best recomputed candidate" % what
    # and against the exact logits, within the two rows' bounds
    if np.all(fin):
        jb = min(range(k), key=lambda i: _order_key(exact[i], int(cand[i])))
        assert exact[j] >= exact[jb] - bound[j] - bound[jb]
    return exact, bound


def test_rescore_lm_head_after_int4_gemv():
    """The 0.5B output projection (151,936 x 896): int4 GEMV stores the
    logits, then the rescore over its fp16 copy; k = 1, 16, 64 and 107 (the
    largest the collection holds at this n); k = 1 is plain greedy."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    W, x = inputs.sweep_matrix("qwen2.5-0.5b", 168, 151936, 896)
    Wd = torch.from_numpy(W).cuda()
    codes, meta = tkq.pack_int4_g128(Wd)
    xd = torch.from_numpy(x).cuda()
    y = tkq.gemv("int4", codes, meta, xd, 151936, 896)
    head16 = W.astype(np.float16)
    hd = Wd.half().contiguous()
    torch.cuda.synchronize()
    y16 = y.cpu().numpy()
    for k in (1, 16, 64, 107):
        tok, cand, cl = _rescore_dev(torch, tkq, y, hd, xd, k, calls=2)
        _check(y16, lambda r: head16[r], x, k, tok, cand, cl, "lm_head k=%d" % k)
        if k == 1:
            assert tok == oref.greedy_token(y16)


@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (8, 8), (9, 2), (100, 64), (1000, 17), (8191, 5),
                                 (8193, 100), (20000, 64), (70001, 33), (10000, 1024)])
@pytest.mark.parametrize("kind", ["normal", "ties", "sorted", "nan", "negzero", "infs", "oneshare", "const"])
def test_rescore_ragged(n, k, kind):
    """Ragged n (partial last chunk, fewer than k non-empty shares), ties,
    NaN of either sign, -0 next to +0 and as the largest value, infinities, ascending logits (many keys collected, sorted rather
    than ranked), the top logits packed into one thread's share, and all
    logits equal (the threshold decided by rows alone; at k = 1024 the
    collection is full)."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    rng = np.random.default_rng((700, n, k, len(kind)))
    K = 264
    if kind == "normal":
        y = (rng.standard_normal(n) * 3).astype(np.float16)
    elif kind == "ties":
        y = np.round(rng.standard_normal(n)).astype(np.float16)
    elif kind == "sorted":
        y = np.sort(rng.standard_normal(n)).astype(np.float16)
    elif kind == "nan":
        y = rng.standard_normal(n).astype(np.float16)
        y[rng.integers(0, n, 1 + n // 50)] = np.nan
        y[rng.integers(0, n, 1 + n // 50)] = -np.nan      # sign bit set
        y[::7] = -0.0
        y[1::7] = 0.0
    elif kind == "negzero":
        y = -np.abs(rng.standard_normal(n)).astype(np.float16)
        y[::5] = -0.0
    elif kind == "infs":
        y = np.full(n, -np.inf, np.float16)
        y[rng.integers(0, n, 3)] = np.inf
    elif kind == "const":
        y = np.full(n, -2.25, np.float16)
    else:
        y = rng.standard_normal(n).astype(np.float16)
        for c in range(3, (n + 7) // 8, 1024):
            y[8 * c:8 * c + 8] = 60000
    head = (rng.standard_normal((n, K)) * 0.05).astype(np.float16)
    x = rng.standard_normal(K).astype(np.float16)
    tok, cand, cl = _rescore(torch, tkq, y, head, x, k, calls=2)
    _check(y, lambda r: head[r], x, k, tok, cand, cl, "%s n=%d k=%d" % (kind, n, k))


def test_rescore_ties_in_recomputed_logits():
    """Equal logits everywhere: the candidates are rows 0..k-1; equal
    recomputed logits go to the smaller row whatever the candidate order."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    n, K, k = 5000, 64, 40
    y = np.full(n, 1.5, np.float16)
    head = np.zeros((n, K), np.float16)
    head[:, 0] = 1.0
    head[[3, 17, 30], 0] = 2.0          # three equal maxima among the candidates
    x = np.ones(K, np.float16)
    tok, cand, cl = _rescore(torch, tkq, y, head, x, k)
    assert list(cand) == list(range(k)) and tok == 3
    _check(y, lambda r: head[r], x, k, tok, cand, cl, "ties")


def test_rescore_changes_the_token_and_non_finite_rows():
    """The rescore picks a candidate other than the stored maximum; a head row
    with +inf gives +inf, one with +inf and -inf gives NaN (ranked first)."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    n, K, k = 3000, 128, 8
    rng = np.random.default_rng(710)
    y = rng.standard_normal(n).astype(np.float16)
    top = np.argsort(-y.astype(np.float64), kind="stable")[:k]
    head = (rng.standard_normal((n, K)) * 0.01).astype(np.float16)
    x = np.ones(K, np.float16)
    head[top[5], :] = 0.5                # exact logit 64: the best candidate, not the stored best
    tok, cand, cl = _rescore(torch, tkq, y, head, x, k)
    assert tok == int(top[5])
    _check(y, lambda r: head[r], x, k, tok, cand, cl, "rescore changes token")
    head[top[2], 3] = np.inf
    tok, cand, cl = _rescore(torch, tkq, y, head, x, k)
    assert tok == int(top[2]) and np.isposinf(cl[2])
    _check(y, lambda r: head[r], x, k, tok, cand, cl, "inf row")
    head[top[6], 4] = -np.inf
    head[top[6], 5] = np.inf
    tok, cand, cl = _rescore(torch, tkq, y, head, x, k)
    assert tok == int(top[6]) and np.isnan(cl[6])
    _check(y, lambda r: head[r], x, k, tok, cand, cl, "nan row")


def test_rescore_maximum_sizes():
    """The largest n at k = 64 (262,144: the collection's capacity) and the
    largest K (2^20) with k = n = 64; heads drawn on the device, only the
    candidate rows copied back."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    for n, K, k in ((262144, 896, 64), (64, 1 << 20, 64), (4096, 1 << 14, 1024 // 8)):
        g = torch.Generator("cuda").manual_seed(720 + n)
        hd = (torch.randn(n, K, generator=g, device="cuda") * 0.02).half()
        y = (torch.randn(n, generator=g, device="cuda") * 2).half()
        xd = torch.randn(K, generator=g, device="cuda").half()
        tok, cand, cl = _rescore_dev(torch, tkq, y, hd, xd, k)
        y16 = y.cpu().numpy()
        x16 = xd.cpu().numpy()
        rows = lambda r: hd[torch.from_numpy(np.asarray(r)).cuda()].cpu().numpy()
        _check(y16, rows, x16, k, tok, cand, cl, "max n=%d K=%d" % (n, K))


# ---- fused: grouped GEMV + head rescore (tkq_gemv_argmax_rescore) ----------

_PACK = {"int4": "pack_int4_g128", "k5": "pack_k5", "tern": "pack_tern_g128", "hier": "pack_int4_hier_g32",
         "int2": "pack_int2_g128", "int3": "pack_int3_g128"}


def _fused(torch, tkq, fmt, mats, target, k, calls=2, Wdev=None):
    """Grouped GEMV of `mats` [(W numpy or None, x numpy)] with the fused
    rescore over `target`; returns (token, cand, cand_logits, stored y of the
    target, head fp16 on the device, x of the target on the device)."""
    items = []
    for i, (W, x) in enumerate(mats):
        Wd = Wdev if (W is None) else torch.from_numpy(W).cuda()
        N, K = Wd.shape
        codes, meta = getattr(tkq, _PACK[fmt])(Wd)
        y = torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
        items.append(dict(codes=codes, meta=meta, x=torch.from_numpy(x).cuda(), y=y, N=N, K=K))
        if i == target:
            head = Wd.half().contiguous()
    batch = tkq.GemvBatch(fmt, items)
    scratch = batch.greedy_scratch()
    outs = []
    for c in range(calls):
        token = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        cand = torch.full((k,), -7, dtype=torch.int32, device="cuda")
        cl = torch.full((k,), float("nan"), dtype=torch.float32, device="cuda")
        scratch.random_(0, 2 ** 62, generator=torch.Generator("cuda").manual_seed(c))   # garbage in the scratch
        batch.run_argmax_rescore(target, head, k, token, scratch, cand=cand, cand_logits=cl)
        torch.cuda.synchronize()
        outs.append((int(token.item()), cand.cpu().numpy(), cl.cpu().numpy()))
    for o in outs[1:]:
        assert o[0] == outs[0][0] and np.array_equal(o[1], outs[0][1])
        assert np.array_equal(o[2].view(np.uint32), outs[0][2].view(np.uint32))
    return outs[0] + (items[target]["y"], head, items[target]["x"])


def _fused_check(torch, tkq, res, k, what):
    """The fused result equals the standalone rescore over the same stored
    logits bit for bit, and both meet the oracle."""
    tok, cand, cl, y, head, xd = res
    t2, c2, l2 = _rescore_dev(torch, tkq, y, head, xd, k)
    assert tok == t2 and np.array_equal(cand, c2), "%s: fused and standalone rescore differ" % what
    assert np.array_equal(cl.view(np.uint32), l2.view(np.uint32)), what
    rows = lambda r: head[torch.from_numpy(np.asarray(r)).cuda()].cpu().numpy()
    _check(y.cpu().numpy(), rows, xd.cpu().numpy(), k, tok, cand, cl, what)


def test_fused_rescore_lm_head():
    """The 0.5B output projection alone (large tiles, then the small tail
    tiles): k = 1, 16, 64, 107; the stored logits equal a plain GEMV's."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    W, x = inputs.sweep_matrix("qwen2.5-0.5b", 168, 151936, 896)
    for k in (1, 16, 64, 107):
        res = _fused(torch, tkq, "int4", [(W, x)], 0, k)
        _fused_check(torch, tkq, res, k, "lm_head k=%d" % k)
        if k == 1:
            codes, meta = tkq.pack_int4_g128(torch.from_numpy(W).cuda())
            yp = tkq.gemv("int4", codes, meta, torch.from_numpy(x).cuda(), 151936, 896)
            torch.cuda.synchronize()
            assert np.array_equal(res[3].cpu().numpy().view(np.uint16), yp.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("fmt", ["int4", "k5", "tern", "hier", "int2", "int3"])
def test_fused_rescore_grouped(fmt):
    """Mixed shapes in one launch, the target first, in the middle and last;
    the other codings' tiles need not start on multiples of 8 rows."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    shapes = [(896, 896), (128, 896), (4864, 896), (896, 4864), (20000, 896)]
    mats = [(inputs.normal_matrix((730, i), n, kk), inputs.normal_vector((731, i), kk))
            for i, (n, kk) in enumerate(shapes)]
    for target, k in ((0, 64), (2, 33), (4, 100), (1, 128)):
        res = _fused(torch, tkq, fmt, mats, target, k)
        _fused_check(torch, tkq, res, k, "%s target %d k=%d" % (fmt, target, k))


@pytest.mark.parametrize("distinct", [1, 3])
def test_fused_rescore_ties_fall_back(distinct):
    """Rows drawn from one or three distinct rows: the stored logits take that
    many values and every tile maximum ties.  With three values the winners'
    rows hold ~8,700 keys at k = 64, which the collection takes; with one,
    every row of the first k - 1 (large) tiles ties, more than the collection
    takes, so the selection starts again from the logits.  Equal recomputed
    logits go to the smallest row."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K = 151936, 896
    rng = np.random.default_rng(740 + distinct)
    base = torch.from_numpy((rng.standard_normal((distinct, K)) * 0.02).astype(np.float32)).cuda()
    pick = torch.from_numpy(rng.integers(0, distinct, N)).cuda()
    Wd = base[pick].contiguous()
    x = inputs.normal_vector(741, K)
    for k in (1, 64, 107):
        res = _fused(torch, tkq, "int4", [(None, x)], 0, k, Wdev=Wd)
        _fused_check(torch, tkq, res, k, "%d-row ties k=%d" % (distinct, k))
        if distinct == 1:
            assert res[0] == 0 and list(res[1]) == list(range(k))


def test_fused_rescore_7b_head():
    """The 7B output projection (152,064 x 3,584, weights drawn on the
    device) in int4 and int4-hier-g32, k = 64: longer head rows in the
    recompute, other tile heights."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K = 152064, 3584
    Wd = inputs.device_normal_matrix(torch, 5196, N, K)
    x = inputs.sweep_x("qwen2.5-7b", 196, K)
    for fmt in ("int4", "hier"):
        res = _fused(torch, tkq, fmt, [(None, x)], 0, 64, Wdev=Wd)
        _fused_check(torch, tkq, res, 64, "7B head %s" % fmt)
    del Wd
    torch.cuda.empty_cache()

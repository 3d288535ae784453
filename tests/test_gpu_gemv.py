"""GPU grouped GEMV against the fp64 oracle: per-row bound for the float
codings, bit-exact for binary; ragged shapes spanning several tiles, grouped
launches of mixed shapes, and the special cases with exact answers."""

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
from helpers import (assert_codes_equal, check_gemv, device_codes_np, gpu_or_skip, oracle_pack,
                     oracle_wdeq)
from oracle import ref as oref

pytestmark = pytest.mark.gpu

MAXK = {"int4": 18944, "k5": 4864, "tern": 18944, "bin": 18944, "hier": 18944, "int2": 18944,
        "int3": 18944}
FLOAT_FMTS = ["int4", "k5", "tern", "hier", "int2", "int3"]


def _shapes(fmt):
    s = [(1, 128), (5, 256), (128, 896), (333, 896), (1000, 4864), (77, 1152), (2049, 384)]
    if fmt == "hier":                       # K % 32 == 0 suffices
        s += [(3, 32), (70, 96), (129, 160), (40, 32 * 593)]
    s.append((300, MAXK[fmt]))
    return s


def _inputs(fmt, N, K, seed):
    if fmt == "bin":
        W = (1 - 2 * np.random.default_rng((seed, 1)).integers(0, 2, (N, K))).astype(np.float32)
        x = (1 - 2 * np.random.default_rng((seed, 2)).integers(0, 2, K)).astype(np.float32)
        return W, x
    return inputs.normal_matrix((seed, N, K), N, K), inputs.normal_vector((seed, 9, K), K)


def _device_pack(torch, tkq, fmt, Wd):
    if fmt == "int4":
        return tkq.pack_int4_g128(Wd)
    if fmt == "k5":
        return tkq.pack_k5(Wd)
    if fmt == "tern":
        return tkq.pack_tern_g128(Wd)
    if fmt == "hier":
        return tkq.pack_int4_hier_g32(Wd)
    if fmt == "int2":
        return tkq.pack_int2_g128(Wd)
    if fmt == "int3":
        return tkq.pack_int3_g128(Wd)
    return tkq.pack_bin(Wd), None


def _items(torch, tkq, fmt, mats):
    items = []
    for W, x in mats:
        N, K = W.shape
        codes, meta = _device_pack(torch, tkq, fmt, torch.from_numpy(W).cuda())
        if fmt == "bin":
            xd = tkq.pack_bin(torch.from_numpy(x).cuda())
            y = torch.full((N,), -7, dtype=torch.int32, device="cuda")
        else:
            xd = torch.from_numpy(x).cuda()
            y = torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
        items.append(dict(codes=codes, meta=meta, x=xd, y=y, N=N, K=K))
    return items


def _check(fmt, W, x, y, codes, meta, what):
    oc, om = oracle_pack(fmt, W)
    assert_codes_equal(fmt, device_codes_np(fmt, codes, meta), (oc, om))
    K = W.shape[1]
    if fmt == "bin":
        xb = oracle_pack("bin", x[None, :])[0][0]
        want = oref.bin_gemv(oc, xb, K)
        got = y.cpu().numpy()
        assert np.array_equal(got, want), "%s: %d rows differ" % (what, int((got != want).sum()))
        return
    w_deq = oracle_wdeq(fmt, oc, om, K)
    check_gemv(y.float().cpu().numpy(), w_deq, x, what)


@pytest.mark.parametrize("fmt", ["int4", "k5", "tern", "bin", "hier", "int2", "int3"])
def test_gemv_single_shapes(fmt):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    for i, (N, K) in enumerate(_shapes(fmt)):
        W, x = _inputs(fmt, N, K, 100 + i)
        (it,) = _items(torch, tkq, fmt, [(W, x)])
        tkq.GemvBatch(fmt, [it]).run()
        torch.cuda.synchronize()
        _check(fmt, W, x, it["y"], it["codes"], it["meta"], "%s %dx%d" % (fmt, N, K))


@pytest.mark.parametrize("fmt", ["int4", "k5", "tern", "bin", "hier", "int2", "int3"])
def test_gemv_grouped_mixed_shapes(fmt):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    mats = [_inputs(fmt, N, K, 200 + i) for i, (N, K) in enumerate(_shapes(fmt))]
    items = _items(torch, tkq, fmt, mats)
    batch = tkq.GemvBatch(fmt, items)
    batch.run()
    torch.cuda.synchronize()
    first = [it["y"].clone() for it in items]
    for (W, x), it in zip(mats, items):
        _check(fmt, W, x, it["y"], it["codes"], it["meta"], "%s grouped %s" % (fmt, W.shape))
    # a second launch gives bit-identical outputs (no races, no state)
    for it in items:
        it["y"].fill_(0)
    batch.run()
    torch.cuda.synchronize()
    for a, it in zip(first, items):
        assert torch.equal(a, it["y"])


@pytest.mark.parametrize("fmt", FLOAT_FMTS)
def test_gemv_unit_vectors_bit_exact(fmt):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K = 300, 896
    W = inputs.normal_matrix((301, N, K), N, K)
    oc, om = oracle_pack(fmt, W)
    w_deq = oracle_wdeq(fmt, oc, om, K)
    codes, meta = _device_pack(torch, tkq, fmt, torch.from_numpy(W).cuda())
    for k in (0, 1, 4, 5, 31, 32, 127, 128, 500, 895):
        e = torch.zeros(K, dtype=torch.float16, device="cuda")
        e[k] = 1
        y = tkq.gemv(fmt, codes, meta, e, N, K)
        torch.cuda.synchronize()
        want = w_deq[:, k].astype(np.float16)
        assert np.array_equal(y.cpu().numpy().view(np.uint16), want.view(np.uint16)), (fmt, k)


@pytest.mark.parametrize("fmt", FLOAT_FMTS)
def test_gemv_exact_zeros(fmt):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K = 130, 896
    W = inputs.normal_matrix((401, N, K), N, K)
    W[7] = 0.0          # zero rows
    W[64] = 0.0
    W[100, :128] = 0.0  # one zero group inside a live row
    codes, meta = _device_pack(torch, tkq, fmt, torch.from_numpy(W).cuda())
    x = torch.from_numpy(inputs.normal_vector(402, K)).cuda()
    y = tkq.gemv(fmt, codes, meta, x, N, K).float().cpu().numpy()
    assert y[7] == 0 and y[64] == 0
    oc, om = oracle_pack(fmt, W)
    check_gemv(y, oracle_wdeq(fmt, oc, om, K), x.cpu().numpy(), fmt)
    y0 = tkq.gemv(fmt, codes, meta, torch.zeros(K, dtype=torch.float16, device="cuda"), N, K)
    torch.cuda.synchronize()
    assert torch.all(y0 == 0)


def test_gemv_bin_all_plus_x():
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    N, K = 257, 4864
    W, _ = inputs.binary_case(N, K)
    bits = tkq.pack_bin(torch.from_numpy(W).cuda())
    xb = torch.zeros(K // 32, dtype=torch.int32, device="cuda")       # all +1
    y = tkq.gemv("bin", bits, None, xb, N, K).cpu().numpy()
    assert np.array_equal(y, K - 2 * (W < 0).sum(axis=1))


# largest K each coding's GEMV accepts (the header's limits), and one past it
MAX_GEMV_K = {"int4": 32768, "hier": 32768, "tern": 32768, "int2": 32768, "int3": 32768, "k5": 16384,
              "bin": 262144}


@pytest.mark.parametrize("fmt", ["int4", "k5", "tern", "bin", "hier", "int2", "int3"])
def test_gemv_max_k(fmt):
    """The longest rows a GEMV takes: 70 rows (ragged tiles) at the maximum K,
    checked against the oracle; K one unit further is refused."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    K = MAX_GEMV_K[fmt]
    W, x = _inputs(fmt, 70, K, 300)
    (it,) = _items(torch, tkq, fmt, [(W, x)])
    tkq.GemvBatch(fmt, [it]).run()
    torch.cuda.synchronize()
    _check(fmt, W, x, it["y"], it["codes"], it["meta"], "%s 70x%d" % (fmt, K))
    unit = 32 if fmt in ("hier", "bin") else 128
    big = dict(it, K=K + unit)
    with pytest.raises(tkq.TkqError):
        tkq.GemvBatch(fmt, [big])


@pytest.mark.parametrize("fmt", FLOAT_FMTS)
@pytest.mark.parametrize("N,K", [(300, 896), (129, 4864), (64, 18944)])
def test_gemv_large_activations(fmt, N, K):
    """Activation channels of 1e3..3e4 on weights at their zero point (and one
    outlier weight per group, heavy-tailed weights): the per-row bound holds,
    i.e. the rounding error follows |w x| and not the activations' size."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    K = min(K, MAXK[fmt])
    W, x = inputs.outlier_case((31, N, K), N, K)
    items = _items(torch, tkq, fmt, [(W, x)])
    tkq.GemvBatch(fmt, items).run()
    torch.cuda.synchronize()
    it = items[0]
    _check(fmt, W, x, it["y"], it["codes"], it["meta"], "%s outliers %dx%d" % (fmt, N, K))


def test_gemv_and_pack_on_a_side_stream():
    """stream= names a stream other than the current one: the packer, the
    single GEMV (whose output and descriptor table the binding allocates) and
    a prepared batch run there and give the current-stream results."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    W, x = _inputs("int4", 333, 896, 41)
    Wd, xd = torch.from_numpy(W).cuda(), torch.from_numpy(x).cuda()
    codes, meta = tkq.pack_int4_g128(Wd)
    y0 = tkq.gemv("int4", codes, meta, xd, 333, 896)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    c2, m2 = tkq.pack_int4_g128(Wd, stream=side)
    ys = [tkq.gemv("int4", c2, m2, xd, 333, 896, stream=side) for _ in range(3)]
    side.synchronize()
    assert torch.equal(c2, codes) and torch.equal(m2, meta)
    for y in ys:
        assert torch.equal(y, y0)
    _check("int4", W, x, y0, codes, meta, "side stream")


@pytest.mark.parametrize("N,K", [(70, 32640), (97, 16256), (33, 128 * 3)])
def test_gemv_int4_odd_group_counts(N, K):
    """int4 rows with an odd number of 128-weight groups: x is held twice in
    LDS and the tile's units pair groups across row ends; K = 32640 is the
    largest LDS footprint a tile can have (x twice plus 32 rows of metadata)."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    W, x = _inputs("int4", N, K, 500 + K // 128)
    (it,) = _items(torch, tkq, "int4", [(W, x)])
    tkq.GemvBatch("int4", [it]).run()
    torch.cuda.synchronize()
    _check("int4", W, x, it["y"], it["codes"], it["meta"], "int4 %dx%d" % (N, K))

"""Full-size workloads in the launch configuration the benchmark times: the
single 896x896 GEMV, the Qwen2.5-0.5B sweep (169 GEMVs in one launch) in the
int4, K5, ternary, int4-hier-g32, int2 and int3 codings, the binary sign
GEMVs, and the Qwen2.5-7B int4 sweep (197 GEMVs).  0.5B: every packed code
and every output row of every matrix against the oracle (row blocks on the
host).  7B (weights drawn on the device): codes and outputs of the first and
last row of every row tile the planner made, plus random rows.  Binary:
every output exact."""

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
from helpers import (assert_codes_equal, check_gemv, device_codes_np, gpu_or_skip, oracle_pack,
                     oracle_wdeq, tile_edge_rows)
from oracle import ref as oref

pytestmark = pytest.mark.gpu

FLOAT_FMTS = ("int4", "k5", "tern", "hier", "int2", "int3")
BLOCK = 16384   # rows per host check block


def _sample_rows(N, i):
    r = np.random.default_rng((77, i)).integers(0, N, 6)
    return np.unique(np.concatenate([[0, N - 1], r]))


def test_single_gemv_896():
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    W, x = inputs.single_gemv_896()
    codes, meta = tkq.pack_int4_g128(torch.from_numpy(W).cuda())
    y = tkq.gemv("int4", codes, meta, torch.from_numpy(x).cuda(), 896, 896)
    torch.cuda.synchronize()
    oc, om = oracle_pack("int4", W)
    assert_codes_equal("int4", device_codes_np("int4", codes, meta), (oc, om))
    check_gemv(y.float().cpu().numpy(), oracle_wdeq("int4", oc, om, 896), x, "896x896")


@pytest.fixture(scope="module")
def sweep05b():
    """Qwen2.5-0.5B sweep: host weights and activations of all 169 matrices."""
    gpu_or_skip()
    return [inputs.sweep_matrix("qwen2.5-0.5b", i, N, K)
            for i, (_, N, K) in enumerate(inputs.sweep_shapes("qwen2.5-0.5b"))]


def _pack_device(tkq, fmt, Wd):
    return {"int4": tkq.pack_int4_g128, "k5": tkq.pack_k5, "tern": tkq.pack_tern_g128,
            "hier": tkq.pack_int4_hier_g32, "int2": tkq.pack_int2_g128, "int3": tkq.pack_int3_g128}[fmt](Wd)


@pytest.mark.parametrize("fmt", FLOAT_FMTS)
def test_sweep_05b(sweep05b, fmt):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    items = []
    for W, x in sweep05b:
        N, K = W.shape
        codes, meta = _pack_device(tkq, fmt, torch.from_numpy(W).cuda())
        y = torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
        items.append(dict(codes=codes, meta=meta, x=torch.from_numpy(x).cuda(), y=y, N=N, K=K))
    assert len(items) == 169
    tkq.GemvBatch(fmt, items).run()
    torch.cuda.synchronize()
    worst = 0.0
    for i, (it, (W, x)) in enumerate(zip(items, sweep05b)):
        N, K = it["N"], it["K"]
        oc, om = oracle_pack(fmt, W)
        assert_codes_equal(fmt, device_codes_np(fmt, it["codes"], it["meta"]), (oc, om))
        y = it["y"].float().cpu().numpy()
        assert np.all(np.isfinite(y))
        if fmt == "hier":                   # one metadata block per matrix: dequantize whole
            worst = max(worst, check_gemv(y, oracle_wdeq(fmt, oc, om, K), x, "%s #%d" % (fmt, i)))
            continue
        for r0 in range(0, N, BLOCK):
            sl = slice(r0, min(N, r0 + BLOCK))
            c = oc[:, sl] if fmt == "int3" else oc[sl]
            wd = oracle_wdeq(fmt, c, om[sl], K)
            worst = max(worst, check_gemv(y[sl], wd, x, "%s #%d rows %d.." % (fmt, i, r0)))
    print("sweep %s: every row of 169 matrices, worst |err|/bound %.3g" % (fmt, worst))


def test_binary_shapes_exact():
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    items, cases = [], []
    for N, K in inputs.BINARY_SHAPES:
        W, x = inputs.binary_case(N, K)
        bits = tkq.pack_bin(torch.from_numpy(W).cuda())
        xb = tkq.pack_bin(torch.from_numpy(x).cuda())
        y = torch.full((N,), -7, dtype=torch.int32, device="cuda")
        items.append(dict(codes=bits, meta=None, x=xb, y=y, N=N, K=K))
        cases.append((W, x))
    tkq.GemvBatch("bin", items).run()
    torch.cuda.synchronize()
    for it, (W, x) in zip(items, cases):
        wb, _ = oracle_pack("bin", W)
        xb, _ = oracle_pack("bin", x[None, :])
        assert_codes_equal("bin", device_codes_np("bin", it["codes"], None), (wb, None))
        want = oref.bin_gemv(wb, xb[0], it["K"])
        assert np.array_equal(it["y"].cpu().numpy(), want)
        assert np.array_equal(want.astype(np.int64), oref.bin_dot(W, x))


def test_sweep_7b_int4():
    """Qwen2.5-7B int4 sweep (197 GEMVs, 3.76 GB packed); weights drawn on the
    device (torch Philox, seed 5000 + i).  Checked rows: the first and last
    row of every row tile of the launch plan, and random rows."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    shapes = inputs.sweep_shapes("qwen2.5-7b")
    items, Ws = [], []
    for i, (_, N, K) in enumerate(shapes):
        Wd = inputs.device_normal_matrix(torch, 5000 + i, N, K)
        codes, meta = tkq.pack_int4_g128(Wd)
        Ws.append(Wd if N * K <= 128 << 20 else None)   # big ones are re-drawn later
        x = torch.from_numpy(inputs.sweep_x("qwen2.5-7b", i, K)).cuda()
        y = torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
        items.append(dict(codes=codes, meta=meta, x=x, y=y, N=N, K=K))
        del Wd
    batch = tkq.GemvBatch("int4", items)
    batch.run()
    torch.cuda.synchronize()
    nrows = 0
    for i, (it, desc) in enumerate(zip(items, batch.descs)):
        rows = np.unique(np.concatenate([tile_edge_rows(desc), _sample_rows(it["N"], i)]))
        rt = torch.from_numpy(rows).cuda()
        Wd = Ws[i] if Ws[i] is not None else inputs.device_normal_matrix(torch, 5000 + i, it["N"], it["K"])
        Wr = Wd[rt].cpu().numpy()
        del Wd
        Ws[i] = None
        oc, om = oracle_pack("int4", Wr)
        assert_codes_equal("int4", device_codes_np("int4", it["codes"][rt], it["meta"][rt]), (oc, om))
        y = it["y"].float().cpu().numpy()
        assert np.all(np.isfinite(y))
        check_gemv(y[rows], oracle_wdeq("int4", oc, om, it["K"]), it["x"].cpu().numpy(),
                   "7b #%d N=%d K=%d" % (i, it["N"], it["K"]))
        nrows += rows.size
    print("7b int4 sweep: %d rows checked (every tile's first and last row)" % nrows)

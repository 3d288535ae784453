"""Full-size workloads in the launch configuration the benchmark times: the
single 896x896 GEMV, the Qwen2.5-0.5B sweep (169 GEMVs in one launch) in the
int4, K5, ternary, int4-hier-g32, int2 and int3 codings, the binary sign GEMVs, and the Qwen2.5-7B int4
sweep (197 GEMVs).  Codes of sampled rows are bit-exact against the oracle's
quantization of the same rows; sampled outputs are within the per-row bound
(binary: every output exact)."""

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
from helpers import (assert_codes_equal, check_gemv, device_codes_np, device_rows_np, gpu_or_skip, oracle_pack,
                     oracle_wdeq)
from oracle import ref as oref

pytestmark = pytest.mark.gpu


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
    """Qwen2.5-0.5B sweep packed in every float coding, with sampled rows."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    shapes = inputs.sweep_shapes("qwen2.5-0.5b")
    packed = {f: [] for f in ("int4", "k5", "tern", "hier", "int2", "int3")}
    samples = []
    for i, (_, N, K) in enumerate(shapes):
        W, x = inputs.sweep_matrix("qwen2.5-0.5b", i, N, K)
        rows = _sample_rows(N, i)
        samples.append((rows, W[rows].copy(), x))
        Wd = torch.from_numpy(W).cuda()
        xd = torch.from_numpy(x).cuda()
        for f, fn in (("int4", tkq.pack_int4_g128), ("k5", tkq.pack_k5), ("tern", tkq.pack_tern_g128),
                      ("hier", tkq.pack_int4_hier_g32), ("int2", tkq.pack_int2_g128),
                      ("int3", tkq.pack_int3_g128)):
            codes, meta = fn(Wd)
            y = torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
            packed[f].append(dict(codes=codes, meta=meta, x=xd, y=y, N=N, K=K))
        del Wd, W
    torch.cuda.synchronize()
    return packed, samples


@pytest.mark.parametrize("fmt", ["int4", "k5", "tern", "hier", "int2", "int3"])
def test_sweep_05b(sweep05b, fmt):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    packed, samples = sweep05b
    items = packed[fmt]
    assert len(items) == 169
    tkq.GemvBatch(fmt, items).run()
    torch.cuda.synchronize()
    worst = 0.0
    for it, (rows, Wr, x) in zip(items, samples):
        y = it["y"].float().cpu().numpy()
        assert np.all(np.isfinite(y))
        oc, om = oracle_pack(fmt, Wr)
        got = device_rows_np(fmt, it["codes"], it["meta"], it["N"], it["K"], rows)
        assert_codes_equal(fmt, got, (oc, om))
        worst = max(worst, check_gemv(y[rows], oracle_wdeq(fmt, oc, om, it["K"]), x,
                                      "%s N=%d K=%d" % (fmt, it["N"], it["K"])))
    print("sweep %s worst |err|/bound %.3g" % (fmt, worst))


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
    device (torch Philox, seed 5000 + i) and sampled rows copied back."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    shapes = inputs.sweep_shapes("qwen2.5-7b")
    items, samples = [], []
    for i, (_, N, K) in enumerate(shapes):
        Wd = inputs.device_normal_matrix(torch, 5000 + i, N, K)
        rows = _sample_rows(N, i)
        samples.append((rows, Wd[torch.from_numpy(rows).cuda()].cpu().numpy()))
        codes, meta = tkq.pack_int4_g128(Wd)
        del Wd
        x = torch.from_numpy(inputs.sweep_x("qwen2.5-7b", i, K)).cuda()
        y = torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
        items.append(dict(codes=codes, meta=meta, x=x, y=y, N=N, K=K))
    tkq.GemvBatch("int4", items).run()
    torch.cuda.synchronize()
    for it, (rows, Wr) in zip(items, samples):
        oc, om = oracle_pack("int4", Wr)
        rt = torch.from_numpy(rows).cuda()
        assert_codes_equal("int4", device_codes_np("int4", it["codes"][rt], it["meta"][rt]), (oc, om))
        y = it["y"].float().cpu().numpy()
        check_gemv(y[rows], oracle_wdeq("int4", oc, om, it["K"]), it["x"].cpu().numpy(),
                   "7b N=%d K=%d" % (it["N"], it["K"]))

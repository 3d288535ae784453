"""GPU packers against the oracle: codes and fp16 metadata bit-exact."""

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
from helpers import assert_codes_equal, device_codes_np, gpu_or_skip, oracle_pack

pytestmark = pytest.mark.gpu

SHAPES = [(1, 128), (7, 256), (37, 896), (130, 4864), (3, 18944)]


def _pack_gpu(fmt, W):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    Wd = torch.from_numpy(np.ascontiguousarray(W)).cuda()
    if fmt == "int4":
        out = tkq.pack_int4_g128(Wd)
    elif fmt == "k5":
        out = tkq.pack_k5(Wd)
    elif fmt == "tern":
        out = tkq.pack_tern_g128(Wd)
    elif fmt == "hier":
        out = tkq.pack_int4_hier_g32(Wd)
    elif fmt == "int2":
        out = tkq.pack_int2_g128(Wd)
    elif fmt == "int3":
        out = tkq.pack_int3_g128(Wd)
    else:
        out = (tkq.pack_bin(Wd), None)
    torch.cuda.synchronize()
    return device_codes_np(fmt, *out)


@pytest.mark.parametrize("fmt", ["int4", "k5", "tern", "bin", "hier", "int2", "int3"])
@pytest.mark.parametrize("shape", SHAPES)
def test_pack_bit_exact(fmt, shape):
    N, K = shape
    W = inputs.normal_matrix((77, N, K), N, K)
    assert_codes_equal(fmt, _pack_gpu(fmt, W), oracle_pack(fmt, W))


def _degenerate_rows():
    rows = []
    rows.append(np.zeros(256, np.float32))                          # all zero
    rows.append(np.full(256, 1e-9, np.float32))                     # scale underflows
    rows.append(np.full(256, -1e-9, np.float32))
    rows.append(np.full(256, -0.3, np.float32))                     # constant negative
    rows.append(np.full(256, 0.7, np.float32))                      # constant positive
    r = np.random.default_rng(3).standard_normal(256).astype(np.float32) * np.float32(1e-6)
    rows.append(r)                                                  # fp16-subnormal scales
    r = np.zeros(256, np.float32)
    r[5] = 100.0                                                    # one outlier
    rows.append(r)
    k = np.tile(np.arange(16), 16).astype(np.float32)
    rows.append((k - 8) / np.float32(16))                           # exact grid
    t = np.zeros(256, np.float32)                                   # rounding ties
    t[0], t[1] = -0.5, 0.4375
    t[2:10] = np.array([0.5, 1.5, -2.5, 3.5, -0.5, 2.5, 7.5, -7.5], np.float32) / 16
    rows.append(t)
    rows.append(np.linspace(-1, 1, 256, dtype=np.float32))
    rows.append(np.array([(-1.0) ** i for i in range(256)], np.float32))  # +-1
    rows.append(np.full(256, -0.0, np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("fmt", ["int4", "k5", "tern", "bin", "hier", "int2", "int3"])
def test_pack_degenerate_groups(fmt):
    W = _degenerate_rows()
    assert_codes_equal(fmt, _pack_gpu(fmt, W), oracle_pack(fmt, W))


def test_pack_single_gemv_896_seed0():
    W, _ = inputs.single_gemv_896()
    assert_codes_equal("int4", _pack_gpu("int4", W), oracle_pack("int4", W))


@pytest.mark.parametrize("K", [32, 96, 4864])
def test_pack_bin_k_multiple_of_32(K):
    W, x = inputs.binary_case(5, K)
    assert_codes_equal("bin", _pack_gpu("bin", W), oracle_pack("bin", W))
    assert_codes_equal("bin", _pack_gpu("bin", x[None, :]), oracle_pack("bin", x[None, :]))


@pytest.mark.parametrize("shape", [(1, 32), (5, 96), (3, 160), (65, 224), (2, 32 * 593)])
def test_pack_hier_k_multiple_of_32(shape):
    """int4-hier-g32 needs only K % 32 == 0: K % 64 == 32 leaves the last
    half-wave of the packer idle; the block padding is written as zeros."""
    N, K = shape
    W = inputs.normal_matrix((78, N, K), N, K)
    W[0, :32] *= np.float32(1e-7)                 # a tiny group beside normal ones
    assert_codes_equal("hier", _pack_gpu("hier", W), oracle_pack("hier", W))


def test_pack_hier_row_scale_guard():
    """Rows whose fp16 row scale underflows (Whetstone, status list): the
    stored d / dmin are 1.0, bit-exact with the oracle, beside normal rows."""
    W = inputs.normal_matrix((79, 6, 256), 6, 256)
    W[1] = 1e-9
    W[2] = -3e-9
    W[3, :] = 0.0
    W[4] *= np.float32(1e-5)
    got = _pack_gpu("hier", W)
    want = oracle_pack("hier", W)
    assert_codes_equal("hier", got, want)
    from oracle import pack as opack
    _, _, d16, dmin16 = opack.unpack_hier_meta(got[1], 6, 256)
    assert np.all(d16[1:4] == 1.0) and np.all(dmin16 != 0)

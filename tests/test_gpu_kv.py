"""GPU low-bit KV cache (tkq_kv_pack, tkq_kv_decode) against oracle.kv: the
paged cache bit-exact with the oracle's quantization of the same K and V, and
the decode output within the derived per-element bound of the fp64 attention
over the dequantized cache.  Shapes: the BitDecoding README's example (batch
1, 32 query and 32 KV heads, head dimension 128, 4096 cached tokens), grouped
queries (2, 4 and 8 query heads per KV head), a single page, batches, and a
peaked attention whose answer is one token's value row."""

import numpy as np
import pytest

from helpers import gpu_or_skip
from oracle import kv as okv

pytestmark = pytest.mark.gpu


def _kv(seed, B, T, Hk):
    r = np.random.default_rng(seed)
    K = r.standard_normal((B, T, Hk, 128)).astype(np.float16)
    V = r.standard_normal((B, T, Hk, 128)).astype(np.float16)
    return K, V


def _q(seed, B, H):
    return np.random.default_rng(seed).standard_normal((B, H, 128)).astype(np.float16)


def _run(torch, tkq, q, K, V):
    cache = tkq.kv_pack(torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda())
    out = tkq.kv_decode(torch.from_numpy(q).cuda(), cache, K.shape[1], 1 / np.sqrt(128))
    torch.cuda.synchronize()
    return cache, out


def _check(q, cache_np, out, what):
    Kd, Vd = okv.dequant_cache(cache_np)
    ref, _ = okv.attention_decode(q.astype(np.float64), Kd, Vd, 1 / np.sqrt(128))
    bound = okv.attention_bound(q.astype(np.float64), Kd, Vd, 1 / np.sqrt(128))
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), what
    ratio = np.abs(got - ref) / bound
    assert ratio.max() <= 1.0, "%s: worst |err|/bound = %g at %s" % (what, ratio.max(),
                                                                     np.unravel_index(ratio.argmax(), ratio.shape))
    return ratio.max()


@pytest.mark.parametrize("B,T,Hk", [(1, 128, 1), (1, 256, 2), (2, 384, 3)])
def test_kv_pack_bit_exact(B, T, Hk):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    K, V = _kv((800, B, T, Hk), B, T, Hk)
    K[0, :128, 0, 5] = 0            # a zero channel (scale guard)
    V[0, 7, 0, :] = 0               # a zero token
    cache = tkq.kv_pack(torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda())
    torch.cuda.synchronize()
    got = cache.cpu().numpy().view(np.uint32).reshape(B, Hk, T // 128, okv.PAGE_WORDS)
    want = okv.pack_cache(K, V)
    assert np.array_equal(got, want), "pages differ at %s" % (np.argwhere(got != want)[:5],)


@pytest.mark.parametrize("B,H,Hk,T", [
    (1, 32, 32, 4096),      # the BitDecoding README example (MHA, 4096 tokens)
    (1, 8, 4, 1024),        # 2 query heads per KV head
    (2, 8, 2, 640),         # 4 per KV head, batch 2, 5 pages
    (1, 16, 2, 2048),       # 8 per KV head
    (1, 28, 4, 1024),       # 7 per KV head (Qwen2.5-7B's attention shape)
    (1, 48, 2, 512),        # 24 per KV head: two workgroups of 12 per KV head
    (1, 32, 2, 1024),       # 16 per KV head: one full matrix-core tile of heads
    (2, 6, 2, 256),         # 3 per KV head (the smallest group on the matrix-core path)
    (1, 1, 1, 128),         # one page
    (1, 32, 32, 32768),     # MHA, 32k tokens: several pages per wave (the other one-head kernel variant)
    (1, 32, 8, 131072),     # GQA, 128k tokens: several pages per wave on the matrix-core path
])
def test_kv_decode_matches_oracle(B, H, Hk, T):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    K, V = _kv((801, B, H, Hk, T), B, T, Hk)
    q = _q((802, B, H, T), B, H)
    cache, out = _run(torch, tkq, q, K, V)
    worst = _check(q, cache.cpu().numpy().view(np.uint32).reshape(B, Hk, T // 128, okv.PAGE_WORDS), out,
                   "B=%d H=%d Hk=%d T=%d" % (B, H, Hk, T))
    print("kv decode B=%d H=%d Hk=%d T=%d worst |err|/bound %.3g" % (B, H, Hk, T, worst))


def test_kv_decode_peaked():
    """One key aligned with the query dominates: the output is that token's
    (dequantized) value row, to fp16 accuracy."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    B, H, Hk, T = 1, 2, 1, 1024
    K, V = _kv(803, B, T, Hk)
    K *= np.float16(0.05)
    q = np.zeros((B, H, 128), np.float16)
    q[0, 0, :] = 1.0
    q[0, 1, :] = -1.0
    K[0, 700, 0, :] = 4.0            # 4 * 128 / sqrt(128) = 45 above the rest for head 0
    K[0, 33, 0, :] = -4.0            # and for head 1
    cache, out = _run(torch, tkq, q, K, V)
    cn = cache.cpu().numpy().view(np.uint32).reshape(B, Hk, T // 128, okv.PAGE_WORDS)
    _check(q, cn, out, "peaked")
    Kd, Vd = okv.dequant_cache(cn)
    got = out.float().cpu().numpy()
    assert np.allclose(got[0, 0], Vd[0, 0, 700], atol=2e-3 * np.abs(Vd[0, 0, 700]).max())
    assert np.allclose(got[0, 1], Vd[0, 0, 33], atol=2e-3 * np.abs(Vd[0, 0, 33]).max())

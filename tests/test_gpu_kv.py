"""GPU low-bit KV cache (tkq_kv_pack, tkq_kv_decode) against oracle.kv: the
paged cache bit-exact with the oracle's quantization of the same K and V, and
the decode output within the per-element bound of the fp64 attention over the
dequantized cache (oracle.kv.attention_bound: the weight GEMV's per-row bound
applied to both products).  Shapes: the BitDecoding README's example (batch
1, 32 query and 32 KV heads, head dimension 128, 4096 cached tokens), grouped
queries (2, 4, 7, 8, 16 and 24 query heads per KV head), a single page,
batches; structural caches that the bound checks page by page (every score
tied and a marker channel per page, so that a page left out, read twice or
read from another head moves an output far beyond the bound), and one peaked
token whose value row is the answer, placed in the last page of the last
split and at page boundaries; query outlier channels (1e3..3e4) on key
channels that dequantize to 0."""

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
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
    ref, probs = okv.attention_decode(q.astype(np.float64), Kd, Vd, 1 / np.sqrt(128))
    bound = okv.attention_bound(q.astype(np.float64), Kd, Vd, 1 / np.sqrt(128), probs=probs)
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


def _cache_np(cache, B, Hk, T):
    return cache.cpu().numpy().view(np.uint32).reshape(B, Hk, T // 128, okv.PAGE_WORDS)


@pytest.mark.parametrize("B,H,Hk,T", [
    (1, 32, 32, 4096),      # one page per wave (the one-head kernel that requests K with the metadata)
    (1, 32, 32, 32768),     # several pages per wave, one head per KV head
    (1, 4, 4, 131072),      # 1024 pages per head: many splits, many pages per wave
    (3, 16, 16, 11264),     # 22 splits per head (just past the in-kernel merge), batch 3
    (1, 1, 1, 262144),      # 512 splits of one head
    (1, 32, 8, 32768),      # matrix-core path (4 query heads per KV head)
    (1, 32, 8, 131072),     # matrix-core path, several pages per wave
    (2, 8, 2, 4096),        # batch 2, 4 query heads per KV head
    (2, 4, 2, 2048),        # batch 2, 2 query heads per KV head
])
def test_kv_decode_page_markers(B, H, Hk, T):
    """Every score ties, so the answer is the plain mean over the cache, and
    each page carries a marker channel (value 15 against 1) that depends on
    the page, the KV head and the sequence.  A decode that leaves out,
    repeats or mixes up a page fails the bound here at every T (the CPU
    tests show it for the oracle with one page dropped or read twice)."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    K, V, q = inputs.kv_marker_case(B, H, Hk, T)
    cache, out = _run(torch, tkq, q, K, V)
    cn = _cache_np(cache, B, Hk, T)
    worst = _check(q, cn, out, "markers B=%d H=%d Hk=%d T=%d" % (B, H, Hk, T))
    # the closed form: channel c of (b, hk) averages 15 over its marker pages, 1 elsewhere
    P = T // 128
    got = out.float().cpu().numpy()
    for b in range(B):
        for h in range(H):
            hk = h // (H // Hk)
            n = np.bincount((np.arange(P) + 37 * hk + 11 * b) % 128, minlength=128)
            want = 1.0 + 14.0 * n / P
            assert np.allclose(got[b, h], want, rtol=4e-3, atol=0), (b, h)
    print("kv markers B=%d H=%d Hk=%d T=%d worst |err|/bound %.3g" % (B, H, Hk, T, worst))


@pytest.mark.parametrize("B,H,Hk,T,t", [
    (1, 2, 1, 1024, 700),
    (1, 32, 32, 4096, 4095),           # last token: last page of the last split
    (1, 32, 32, 32768, 32767),
    (1, 32, 32, 32768, 16384),         # first token of a page in the middle
    (1, 32, 8, 32768, 32767),          # matrix-core path
    (1, 32, 8, 131072, 131071),
    (1, 32, 8, 131072, 65535),         # last token of the page before the middle
    (1, 4, 4, 131072, 131071),
])
def test_kv_decode_peaked(B, H, Hk, T, t):
    """One key aligned with the query dominates every head (score ~45 above
    the rest): the output is that token's dequantized value row."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    K, V, q = inputs.kv_peaked_case(B, H, Hk, T, t)
    cache, out = _run(torch, tkq, q, K, V)
    cn = _cache_np(cache, B, Hk, T)
    _check(q, cn, out, "peaked B=%d H=%d Hk=%d T=%d t=%d" % (B, H, Hk, T, t))
    got = out.float().cpu().numpy()
    for hk in range(Hk):
        page = okv.unpack_page(cn[0, hk, t // 128])[1][t % 128]
        for h in range(hk * (H // Hk), (hk + 1) * (H // Hk)):
            assert np.allclose(got[0, h], page, rtol=0, atol=2e-3 * np.abs(page).max()), (h, t)


def _run_varlen(torch, tkq, q, K, V, lens, workspace=None):
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cache = tkq.kv_pack(torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), seqlens=lt)
    out = tkq.kv_decode(torch.from_numpy(q).cuda(), cache, K.shape[1], 1 / np.sqrt(128), seqlens=lt,
                        workspace=workspace)
    torch.cuda.synchronize()
    return cache, out


def _check_varlen(q, cn, out, lens, what):
    Kd, Vd = okv.dequant_cache(cn)
    sm = 1 / np.sqrt(128)
    ref, probs = okv.attention_decode(q.astype(np.float64), Kd, Vd, sm, lens)
    bound = okv.attention_bound(q.astype(np.float64), Kd, Vd, sm, probs=probs, lens=lens)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), "%s: %d elements outside the bound, first at %s" % (
        what, int(bad.sum()), np.argwhere(bad)[0])
    with np.errstate(divide="ignore", invalid="ignore"):
        return float(np.nanmax(np.where(bound > 0, err / bound, 0.0)))


@pytest.mark.parametrize("B,H,Hk,T", [
    (1, 32, 32, 4096),      # one page per wave, merged in the kernel
    (1, 32, 32, 32768),     # several pages per wave, merge launch
    (1, 32, 8, 32768),      # grouped queries on the matrix cores
    (2, 28, 4, 1024),
])
def test_kv_decode_query_outliers(B, H, Hk, T):
    """Query channels of 1e3..3e4 on key channels that dequantize to 0: the
    per-element bound holds (the products are exact small integers times q',
    so the large channels contribute exactly 0 to the scores)."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    K, V, q = inputs.kv_outlier_case(B, H, Hk, T)
    cache, out = _run(torch, tkq, q, K, V)
    cn = cache.cpu().numpy().view(np.uint32).reshape(B, Hk, T // 128, okv.PAGE_WORDS)
    _check(q, cn, out, "outliers B%d H%d Hk%d T%d" % (B, H, Hk, T))


def test_kv_pack_varlen_bit_exact():
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    B, T, Hk, lens = 4, 512, 2, [1, 200, 512, 0]
    K, V = _kv((805, B, T, Hk), B, T, Hk)
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cache = tkq.kv_pack(torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), seqlens=lt)
    torch.cuda.synchronize()
    got = _cache_np(cache, B, Hk, T)
    want = okv.pack_cache(K, V, lens)
    assert np.array_equal(got, want), "pages differ at %s" % (np.argwhere(got != want)[:5],)


@pytest.mark.parametrize("B,H,Hk,T,lens", [
    (4, 32, 32, 4096, [4096, 1000, 129, 1]),      # MHA, partial pages, a single token
    (3, 32, 8, 32768, [32768 - 77, 5000, 0]),     # matrix-core path; an empty sequence
    (2, 4, 4, 131072, [131071, 70001]),           # many splits, lengths inside a split
    (2, 16, 2, 2048, [2047, 640]),                # 8 query heads per KV head
    (2, 6, 2, 384, [383, 2]),                     # 3 per KV head (smallest matrix-core group)
])
def test_kv_decode_varlen_matches_oracle(B, H, Hk, T, lens):
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    K, V = _kv((806, B, H, Hk, T), B, T, Hk)
    q = _q((807, B, H, T), B, H)
    cache, out = _run_varlen(torch, tkq, q, K, V, lens)
    cn = _cache_np(cache, B, Hk, T)
    worst = _check_varlen(q, cn, out, lens, "varlen B=%d H=%d Hk=%d T=%d lens=%s" % (B, H, Hk, T, lens))
    for b, n in enumerate(lens):
        if n == 0:
            assert not out[b].float().abs().sum().item(), "empty sequence must give 0"
    print("kv varlen B=%d H=%d Hk=%d T=%d worst |err|/bound %.3g" % (B, H, Hk, T, worst))


@pytest.mark.parametrize("B,H,Hk,T,lens", [
    (2, 8, 8, 4096, [4000, 333]),
    (1, 32, 8, 32768, [32768 - 100]),
])
def test_kv_decode_varlen_page_markers(B, H, Hk, T, lens):
    """Page markers with lengths that end inside a page: the answer is the
    mean over each sequence's valid tokens only."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    K, V, q = inputs.kv_marker_case(B, H, Hk, T)
    cache, out = _run_varlen(torch, tkq, q, K, V, lens)
    _check_varlen(q, _cache_np(cache, B, Hk, T), out, lens, "varlen markers %s" % (lens,))
    got = out.float().cpu().numpy()
    for b, n in enumerate(lens):
        for h in range(H):
            hk = h // (H // Hk)
            pages = np.arange(n) // 128
            cnt = np.bincount((pages + 37 * hk + 11 * b) % 128, minlength=128)
            assert np.allclose(got[b, h], 1.0 + 14.0 * cnt / n, rtol=4e-3, atol=0), (b, h)


def test_kv_decode_reuses_its_workspace():
    """Consecutive decodes on one workspace zeroed once (each call leaves its
    arrival counters at zero), a smaller configuration after a larger one,
    and a larger one again after re-zeroing: every result matches the
    oracle."""
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    ws = tkq.kv_workspace(2, 32, 8, 8192, "cuda")
    runs = [(2, 32, 8, 8192, [8192, 3000]), (2, 32, 8, 8192, [100, 8000]), (1, 8, 8, 2048, [2048]),
            "zero", (2, 32, 8, 8192, [5000, 1])]
    for i, r in enumerate(runs):
        if r == "zero":
            ws.zero_()
            continue
        B, H, Hk, T, lens = r
        K, V = _kv((808, i), B, T, Hk)
        q = _q((809, i), B, H)
        cache, out = _run_varlen(torch, tkq, q, K, V, lens, workspace=ws)
        _check_varlen(q, _cache_np(cache, B, Hk, T), out, lens, "reuse %d" % i)

"""Low-bit KV cache for decode attention (test infrastructure only).

BitDecoding (the BitDecoding README, usage example): the KV cache of a
long-context decode is stored with 4-bit codes in groups of 128, K quantized
per channel ("k-channel": one scale/zero per channel for every 128 tokens)
and V per token (one scale/zero per token for every 128 channels), head
dimension 128; one decode step attends a single query token over the whole
cache:  out[h] = softmax(scale * q[h] . K^T) . V  with the query head h
reading the KV head h // (H / H_k).

Readings taken where the page is silent:
* The 4-bit quantizer is the same asymmetric round-to-nearest as the int4
  g128 weights (oracle.quant.quantize_int4_g128): per group lo = min(min, 0),
  hi = max(max, 0), s = fp16((hi - lo) / 15), integer zero-point z; a K group
  is one channel over the 128 tokens of a page, a V group is one token over
  its 128 channels.
* Storage is paged: the cache of one (batch, KV head) is a sequence of
  pages of 128 tokens, each page PAGE_BYTES long:
    K codes  uint32 [128 tokens][16]   nibble c of token t: word t*16 + c//8,
                                       bits 4*(c%8)            (8192 bytes)
    V codes  uint32 [128 channels][16] nibble t of channel c: word c*16 + t//8,
                                       bits 4*(t%8)            (8192 bytes)
    K meta   uint32 [128 channels]     half2 {scale, zero} per channel (512)
    V meta   uint32 [128 tokens]       half2 {scale, zero} per token   (512)
  and the cache tensor is [B][H_k][pages][PAGE_BYTES].  V codes are stored
  channel-major so that the value product, like the scores, reads whole
  rows front to back.
* The cache's capacity T is a multiple of 128 (whole pages).  Sequences of
  a batch may have their own lengths len[b] <= T (the README's usage passes
  per-sequence cached lengths): tokens t >= len[b] are packed as zeros and
  take no part in the attention.  A K group (one channel over a page)
  spans 0 anyway, so zeros in place of the missing tokens leave its scale
  and zero-point those of the valid tokens.  A sequence of length 0 has
  output 0.

The attention itself is the plain definition in fp64 from the dequantized
cache.  Its tolerance (attention_bound) is not given by the page; it is
derived from the per-row bound the weight GEMV is held to (the scores and
the output are both GEMVs over the dequantized cache), carried exactly
through the softmax; see that function.
"""

import numpy as np

from . import pack as _pack
from . import quant as _quant
from .ref import TOL

D = 128            # head dimension
PAGE = 128         # tokens per page
PAGE_WORDS = (8192 + 8192 + 512 + 512) // 4
PAGE_BYTES = PAGE_WORDS * 4
_KC, _VC, _KM, _VM = 0, 2048, 4096, 4224   # word offsets of the four parts


def quantize_page(Kp, Vp):
    """One page: Kp, Vp fp16/fp32 [128 tokens][128 channels] ->
    (k_codes [t][c] uint8, k_s fp16 [c], k_z fp16 [c],
     v_codes [t][c] uint8, v_s fp16 [t], v_z fp16 [t]).
    K groups are channels (rows of Kp^T), V groups are tokens (rows of Vp)."""
    Kp = np.asarray(Kp, dtype=np.float32)
    Vp = np.asarray(Vp, dtype=np.float32)
    if Kp.shape != (PAGE, D) or Vp.shape != (PAGE, D):
        raise ValueError("a page is [128 tokens][128 channels]")
    kq, ks, kz = _quant.quantize_int4_g128(np.ascontiguousarray(Kp.T))   # [c][t], per channel
    vq, vs, vz = _quant.quantize_int4_g128(Vp)                           # [t][c], per token
    return kq.T.copy(), ks[:, 0], kz[:, 0], vq, vs[:, 0], vz[:, 0]


def pack_page(k_codes, k_s, k_z, v_codes, v_s, v_z):
    """Quantized page -> uint32 [PAGE_WORDS] in the layout above."""
    out = np.zeros(PAGE_WORDS, dtype=np.uint32)
    out[_KC:_KC + 2048] = _pack.pack_int4(np.asarray(k_codes)).reshape(-1)        # rows = tokens
    out[_VC:_VC + 2048] = _pack.pack_int4(np.asarray(v_codes).T).reshape(-1)      # rows = channels
    out[_KM:_KM + 128] = _pack.pack_int4_meta(np.asarray(k_s)[:, None], np.asarray(k_z)[:, None])[:, 0]
    out[_VM:_VM + 128] = _pack.pack_int4_meta(np.asarray(v_s)[:, None], np.asarray(v_z)[:, None])[:, 0]
    return out


def unpack_page(words):
    """uint32 [PAGE_WORDS] -> dequantized (K [t][c], V [t][c]) in fp64."""
    words = np.asarray(words, dtype=np.uint32)
    kq = _pack.unpack_int4(words[_KC:_KC + 2048].reshape(PAGE, 16), D).astype(np.float64)      # [t][c]
    vq = _pack.unpack_int4(words[_VC:_VC + 2048].reshape(D, 16), PAGE).astype(np.float64).T    # [t][c]
    ks, kz = _pack.unpack_int4_meta(words[_KM:_KM + 128])
    vs, vz = _pack.unpack_int4_meta(words[_VM:_VM + 128])
    K = (kq - kz.astype(np.float64)[None, :]) * ks.astype(np.float64)[None, :]
    V = (vq - vz.astype(np.float64)[:, None]) * vs.astype(np.float64)[:, None]
    return K, V


def pack_cache(K, V, lens=None):
    """K, V [B][T][H_k][128] (token-major, as a decoder writes them) ->
    cache uint32 [B][H_k][T/128][PAGE_WORDS].  lens [B] (optional): tokens at
    or past lens[b] are packed as zeros."""
    K = np.asarray(K)
    V = np.asarray(V)
    B, T, Hk, d = K.shape
    if d != D or T % PAGE:
        raise ValueError("head dimension 128 and whole pages of 128 tokens")
    if lens is not None:
        K = K.copy()
        V = V.copy()
        for b in range(B):
            n = int(np.clip(lens[b], 0, T))
            K[b, n:] = 0
            V[b, n:] = 0
    out = np.zeros((B, Hk, T // PAGE, PAGE_WORDS), dtype=np.uint32)
    for b in range(B):
        for h in range(Hk):
            for p in range(T // PAGE):
                sl = slice(PAGE * p, PAGE * (p + 1))
                out[b, h, p] = pack_page(*quantize_page(K[b, sl, h], V[b, sl, h]))
    return out


def dequant_cache(cache):
    """cache uint32 [B][H_k][P][PAGE_WORDS] -> (K, V) fp64 [B][H_k][T][128]."""
    cache = np.asarray(cache, dtype=np.uint32)
    B, Hk, P, _ = cache.shape
    K = np.zeros((B, Hk, P * PAGE, D))
    V = np.zeros((B, Hk, P * PAGE, D))
    for b in range(B):
        for h in range(Hk):
            for p in range(P):
                K[b, h, PAGE * p:PAGE * (p + 1)], V[b, h, PAGE * p:PAGE * (p + 1)] = unpack_page(cache[b, h, p])
    return K, V


def attention_decode(q, K, V, sm_scale, lens=None):
    """One decode step: q [B][H][128], K, V [B][H_k][T][128] (fp64 values)
    -> (out [B][H][128], p [B][H][T]) in fp64: softmax(sm_scale q.K^T) V,
    query head h reading KV head h // (H / H_k), over the first lens[b]
    tokens of sequence b (all T without lens; none: out 0, p 0)."""
    q = np.asarray(q, dtype=np.float64)
    B, H, _ = q.shape
    Hk, T = K.shape[1], K.shape[2]
    if H % Hk:
        raise ValueError("query heads must be a multiple of KV heads")
    G = H // Hk
    out = np.zeros((B, H, D))
    probs = np.zeros((B, H, T))
    for b in range(B):
        n = T if lens is None else int(np.clip(lens[b], 0, T))
        if n == 0:
            continue
        for h in range(H):
            s = sm_scale * (K[b, h // G, :n] @ q[b, h])
            e = np.exp(s - s.max())
            p = e / e.sum()
            probs[b, h, :n] = p
            out[b, h] = p @ V[b, h // G, :n]
    return out, probs


def attention_bound(q, K, V, sm_scale, eps=TOL, probs=None, lens=None):
    """Per output element tolerance [B][H][128] of a decode step.

    Reading (the BitDecoding page states none): single-query attention is
    two GEMVs over the dequantized cache, the scores s = sm_scale K q and the
    output o = V^T p, and each is held to the per-row bound of the weight
    GEMV, |err| <= eps * sum |w x| with eps = 2e-3.  So
      score error   |ds_t| <= eps * A_t,  A_t = sm_scale * sum_c |q_c K_tc|;
      softmax       with d = max_t |ds_t|, every p_t moves by a factor in
                    [exp(-2d), exp(2d)] (numerator and denominator each by
                    exp(+-d) at most);
      output        the value GEMV over the perturbed p adds eps * sum_t
                    p'_t |V_tc| <= eps * exp(2d) * sum_t p_t |V_tc|;
    hence, exactly (no first-order step),
      |out_c - ref_c| <= ((1 + eps) * exp(2 eps max_t A_t) - 1)
                         * sum_t p_t |V_tc|.
    A kernel's own roundings (fp16 query and probability scaling, fp32 sums,
    the fp16 store) have to fit inside these two per-GEMV budgets.
    `probs` (from attention_decode) may be passed to skip recomputing them;
    lens as in attention_decode (A_t over the valid tokens only)."""
    q = np.asarray(q, dtype=np.float64)
    B, H, _ = q.shape
    Hk = K.shape[1]
    G = H // Hk
    T = K.shape[2]
    if probs is None:
        _, probs = attention_decode(q, K, V, sm_scale, lens)
    bound = np.zeros((B, H, D))
    for b in range(B):
        n = T if lens is None else int(np.clip(lens[b], 0, T))
        if n == 0:
            continue
        for h in range(H):
            A = sm_scale * (np.abs(K[b, h // G, :n]) @ np.abs(q[b, h]))
            factor = (1.0 + eps) * np.exp(2.0 * eps * A.max()) - 1.0
            bound[b, h] = factor * (probs[b, h, :n] @ np.abs(V[b, h // G, :n]))
    return bound

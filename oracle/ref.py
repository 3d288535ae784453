"""Dequantization and the fp64 GEMV / GEMM definitions (test infrastructure only).

The method computes ``y = dequant(W_q) . x`` for a given packed W (Whetstone,
"The one fact that shapes everything": at batch 1 every weight is read once
and used for one multiply-add).  Up to rounding order this has a plain
definition, so the oracle is that definition in fp64: dequantize the stored
codes with the stored fp16 metadata (exact in fp64), then a plain matrix-vector
(or matrix-matrix) product.

Tolerance (per row): |y - y_ref| <= 2e-3 * sum_k |w_deq[n,k] * x[k]|.  The
prefill GEMM uses the entry-wise analogue over its k-sum.
"""

import numpy as np

from . import pack as _pack

GROUP = 128
TOL = 2e-3


# --- dequantization ----------------------------------------------------------

def _expand_groups(per_group, K):
    return np.repeat(np.asarray(per_group, dtype=np.float64), GROUP, axis=1)[:, :K]


def dequant_int4(codes, meta, K):
    """w = s * (q - z) per 128-group (Whetstone, "What the weights can actually
    survive": one fp16 scale and one fp16 zero-point per group).  Exact in fp64."""
    q = _pack.unpack_int4(codes, K).astype(np.float64)
    s, z = _pack.unpack_int4_meta(meta)
    return _expand_groups(s, K) * (q - _expand_groups(z, K))


def dequant_int2(codes, meta, K):
    """w = s * (q - z) per 128-group, q in 0..3 (Whetstone, "int2 g128": the
    int4 g128 metadata with 2-bit codes).  Exact in fp64."""
    q = _pack.unpack_int2(codes, K).astype(np.float64)
    s, z = _pack.unpack_int4_meta(meta)
    return _expand_groups(s, K) * (q - _expand_groups(z, K))


def dequant_int3(codes, meta, K):
    """w = s * (q - z) per 128-group, q in 0..7 (Whetstone, "int3 g128": the
    int4 g128 metadata with 3-bit codes).  Exact in fp64."""
    q = _pack.unpack_int3(codes, K).astype(np.float64)
    s, z = _pack.unpack_int4_meta(meta)
    return _expand_groups(s, K) * (q - _expand_groups(z, K))


def dequant_int4_hier(codes, meta, N, K):
    """w = d * sc * q - dmin * mi per 32-group (Whetstone, quantizer table,
    "group 32 with hierarchical scale metadata", read as Q4_K-style two-level
    scales; see quant.quantize_int4_hier_g32).  Exact in fp64."""
    q = _pack.unpack_int4(codes, K).astype(np.float64)
    sc, mi, d16, dmin16 = _pack.unpack_hier_meta(meta, N, K)
    step = d16.astype(np.float64)[:, None] * sc.astype(np.float64)
    off = dmin16.astype(np.float64)[:, None] * mi.astype(np.float64)
    return np.repeat(step, 32, axis=1) * q - np.repeat(off, 32, axis=1)


def k5_trits(c):
    """Five balanced trits of a K5 byte (TKintegers K5, "What is K5?").

    The base-3 digits d_0..d_4 of c (least significant first), shifted to
    t_i = d_i - 1 in {-1, 0, +1}.  Returns int8 [..., 5]."""
    c = np.asarray(c, dtype=np.int64)
    digits = []
    rest = c.copy()
    for _ in range(5):
        digits.append(rest % 3)
        rest = rest // 3
    return (np.stack(digits, axis=-1) - 1).astype(np.int8)


def k5_value(c):
    """Integer value of a K5 code: sum_i t_i * 3**i over its five trits."""
    t = k5_trits(c).astype(np.int64)
    return (t * (3 ** np.arange(5, dtype=np.int64))).sum(axis=-1)


def dequant_k5(codes, scale16):
    """w = s * value(c) with value(c) from the five balanced trits of c (the
    value of each of the 256 byte values is tabulated once from k5_value)."""
    codes = np.asarray(codes, dtype=np.uint8)
    K = codes.shape[1]
    table = k5_value(np.arange(256)).astype(np.float64)
    return _expand_groups(scale16, K) * table[codes]


def dequant_tern(codes, scale16, K):
    """w = s * (code - 1) per 128-group; code 0/1/2 stands for t = -1/0/+1."""
    c = _pack.unpack_tern(codes, K).astype(np.float64)
    return _expand_groups(scale16, K) * (c - 1.0)


# --- float products ----------------------------------------------------------

def gemv(w_deq, x):
    """y[n] = sum_k w_deq[n,k] * x[k] in fp64 (the plain definition)."""
    return np.asarray(w_deq, dtype=np.float64) @ np.asarray(x, dtype=np.float64)


def gemv_bound(w_deq, x):
    """Per-row tolerance 2e-3 * sum_k |w_deq[n,k] * x[k]| (fp64)."""
    return TOL * (np.abs(np.asarray(w_deq, dtype=np.float64))
                  @ np.abs(np.asarray(x, dtype=np.float64)))


def gemm(X, w_deq):
    """Y[m,n] = sum_k X[m,k] * w_deq[n,k] in fp64 (prefill: X . W_deq^T)."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(w_deq, dtype=np.float64).T


def gemm_bound(X, w_deq):
    """Entry-wise tolerance 2e-3 * sum_k |X[m,k] * w_deq[n,k]|."""
    return TOL * (np.abs(np.asarray(X, dtype=np.float64))
                  @ np.abs(np.asarray(w_deq, dtype=np.float64)).T)


def check_within(y, y_ref, bound):
    """(ok, worst |err|/bound).  A zero bound requires an exact match."""
    err = np.abs(np.asarray(y, dtype=np.float64) - np.asarray(y_ref, dtype=np.float64))
    bound = np.asarray(bound, dtype=np.float64)
    ok = bool(np.all(err <= bound))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                         np.where(err > 0, np.inf, 0.0))
    return ok, float(ratio.max()) if ratio.size else 0.0


# --- binary ------------------------------------------------------------------

def bin_dot(a_pm1, b_pm1):
    """Integer dot product of {-1,+1} vectors (the quantity the identity gives)."""
    return np.asarray(a_pm1, dtype=np.int64) @ np.asarray(b_pm1, dtype=np.int64)


def bin_gemv(w_words, x_words, K):
    """y[n] = K - 2 * popcount(W[n] XOR x) (Whetstone, "Measured hardware facts",
    the XOR-popcount identity for {-1,+1} vectors packed as bits {1,0}).

    w_words uint32 [N][K/32], x_words uint32 [K/32]; returns int32 [N]."""
    w = np.asarray(w_words, dtype=np.uint32)
    x = np.asarray(x_words, dtype=np.uint32)
    pc = np.bitwise_count(w ^ x[None, :]).astype(np.int64).sum(axis=1)
    return (np.int64(K) - 2 * pc).astype(np.int32)


def greedy_token(y):
    """Greedy decoding's choice from one vector of logits (Whetstone README,
    status list: greedy selection stays on the GPU): the index of the largest
    value, the first such index on ties, with -0 and +0 equal.  A plain scan.
    The comparison is on the values as given (the stored fp16 logits of the
    GEMV, or the int32 outputs of the binary coding).

    NaN (the pages are silent; a logit is NaN only when an input is): every
    NaN counts as larger than any number, +inf included, so the first NaN
    wins -- the convention of numpy's argmax."""
    vals = np.asarray(y).astype(np.float64).ravel()
    if vals.size == 0:
        raise ValueError("empty vector")
    best = 0
    for i in range(1, vals.size):
        if np.isnan(vals[best]):
            break
        if np.isnan(vals[i]) or vals[i] > vals[best]:
            best = i
    return best

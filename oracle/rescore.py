"""Greedy selection with head rescore (test infrastructure only).

Whetstone README, "New in 0.6.0" (the --head-rescore item): besides the
quantized output projection, an fp16 copy of it is kept, and only the logits
that decide the token are computed again from that copy, so the token comes
close to what an fp16 output projection would choose while each token still
streams only the quantized projection.

The pages give neither the number of logits computed again nor how they are
picked.  Reading taken here: the candidates are the k largest stored
(quantized) logits, in the order greedy selection uses (value; every NaN
above every number; on equal values the smaller row first); each
candidate's logit is computed again as the dot product of its fp16 row of
the output projection with x; the token is the candidate whose recomputed
logit is largest, by that same order.  k is the caller's choice.

The recomputed logit has a plain definition (a dot product of fp16 numbers),
so the oracle computes it exactly, in fp64.  This module imports nothing
from the HIP path.
"""

import numpy as np

U32 = 2.0 ** -24  # unit roundoff of fp32


def _order_key(v, i):
    # NaN first, then larger values, then smaller rows (-0 == +0 as floats)
    return (0, 0.0, i) if np.isnan(v) else (1, -v, i)


def candidates(logits, k):
    """Rows of the k largest stored logits, largest first, in the order of
    greedy selection (NaN above every number, smaller row first on ties)."""
    vals = np.asarray(logits).astype(np.float64).ravel()
    n = vals.size
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= len(logits)")
    order = sorted(range(n), key=lambda i: _order_key(vals[i], i))
    return np.array(order[:k], dtype=np.int64)


def recompute(head, x, rows):
    """Exact (fp64) logits of the given rows: sum_j head[row, j] * x[j] over
    fp16 head rows and fp16 x (every fp16 value is exact in fp64; the sums
    of the test sizes are exact to fp64 rounding)."""
    W = np.asarray(head)[np.asarray(rows)].astype(np.float64)
    return W @ np.asarray(x).astype(np.float64)


def head_rescore(logits, head, x, k):
    """(token, candidate rows, their exact recomputed logits).

    logits: the stored logits of the quantized output projection, [N];
    head: the fp16 copy of the output projection, [N][K]; x: fp16 [K]."""
    cand = candidates(logits, k)
    exact = recompute(head, x, cand)
    best = min(range(len(cand)), key=lambda j: _order_key(exact[j], int(cand[j])))
    return int(cand[best]), cand, exact


def recompute_bound(head, x, rows):
    """Tolerance for an fp32 evaluation of the recomputed logits: fp16 x fp16
    products are exact in fp32, and any order of K - 1 fp32 additions stays
    within gamma_(K-1) * sum_j |w_j x_j| of the exact sum, with
    gamma_n = n u / (1 - n u), u = 2^-24 (the standard bound for
    floating-point summation in any order)."""
    W = np.asarray(head)[np.asarray(rows)].astype(np.float64)
    xa = np.abs(np.asarray(x).astype(np.float64))
    n = max(W.shape[1] - 1, 1)
    gamma = n * U32 / (1.0 - n * U32)
    return gamma * (np.abs(W) @ xa)

"""Pins of oracle.rescore (greedy selection with head rescore).

* The candidate list equals selection by repeated greedy choice (take the
  greedy token, remove it, repeat), a different procedure that shares only
  the already pinned greedy rule.
* k = 1 reduces to plain greedy selection over the stored logits.
* k = N reduces to the argmax of the full exact product head . x (numpy's
  first-occurrence argmax over the whole matrix-vector product).
* Hand cases: rescoring changes the token; the true maximum outside the
  candidates is not found; equal recomputed logits go to the smaller row
  whatever the candidate order; NaN logits are candidates first.
* The fp32 tolerance holds for sequential and pairwise fp32 sums of
  cancelling terms, and is far below one dropped term.
"""

import numpy as np
import pytest

from oracle import ref, rescore


def _greedy_repeated(logits, k):
    vals = np.asarray(logits)
    left = list(range(vals.size))
    out = []
    for _ in range(k):
        j = ref.greedy_token(vals[left])
        out.append(left.pop(j))
    return out


@pytest.mark.parametrize("seed,n,k", [(1, 40, 5), (2, 300, 16), (3, 2049, 32), (4, 7, 7)])
def test_candidates_match_repeated_greedy(seed, n, k):
    rng = np.random.default_rng(seed)
    y = np.round(rng.standard_normal(n) * 3).astype(np.float16)   # many ties
    y[rng.integers(0, n, 1 + n // 40)] = np.nan
    y[rng.integers(0, n, 2)] = -0.0
    assert list(rescore.candidates(y, k)) == _greedy_repeated(y, k)


def test_k1_is_greedy():
    rng = np.random.default_rng(7)
    for n in (1, 9, 500):
        y = (rng.standard_normal(n) * 4).astype(np.float16)
        head = rng.standard_normal((n, 16)).astype(np.float16)
        x = rng.standard_normal(16).astype(np.float16)
        tok, cand, _ = rescore.head_rescore(y, head, x, 1)
        assert tok == ref.greedy_token(y) and list(cand) == [tok]


def test_k_equals_n_is_full_argmax():
    rng = np.random.default_rng(8)
    for n in (3, 50, 257):
        # small integers: exact products, frequent ties in the exact logits
        head = rng.integers(-3, 4, (n, 24)).astype(np.float16)
        x = rng.integers(-2, 3, 24).astype(np.float16)
        y = (rng.standard_normal(n)).astype(np.float16)
        tok, cand, exact = rescore.head_rescore(y, head, x, n)
        full = head.astype(np.float64) @ x.astype(np.float64)
        assert tok == int(np.argmax(full))
        assert sorted(cand) == list(range(n))
        assert np.array_equal(exact, full[cand])


def _rows(values, K=8):
    """fp16 head whose row r . ones(K) equals values[r] (value in column 0)."""
    h = np.zeros((len(values), K), np.float16)
    h[:, 0] = values
    return h, np.ones(K, np.float16)


def test_rescore_changes_token():
    y = np.array([1.0, 3.0, 2.0, 2.5], np.float16)     # quantized: row 1 first
    head, x = _rows([10.0, 1.0, 2.0, 0.0])             # exact: row 0 largest
    tok, cand, exact = rescore.head_rescore(y, head, x, 2)
    assert list(cand) == [1, 3] and list(exact) == [1.0, 0.0] and tok == 1   # row 0 not a candidate
    tok, cand, _ = rescore.head_rescore(y, head, x, 3)
    assert list(cand) == [1, 3, 2] and tok == 2
    tok, _, _ = rescore.head_rescore(y, head, x, 4)
    assert tok == 0


def test_ties_and_nan():
    y = np.array([0.0, 0.0, 1.0, 0.0, 0.0, 5.0], np.float16)
    head, x = _rows([0.0, 0.0, 4.0, 0.0, 0.0, 4.0])
    tok, cand, _ = rescore.head_rescore(y, head, x, 2)
    assert list(cand) == [5, 2] and tok == 2            # equal recomputed: smaller row
    tok, cand, _ = rescore.head_rescore(y, head, x, 4)
    assert list(cand) == [5, 2, 0, 1]                   # equal logits: smaller rows first
    y2 = y.copy()
    y2[4] = np.nan
    tok, cand, _ = rescore.head_rescore(y2, head, x, 2)
    assert list(cand) == [4, 5] and tok == 5            # NaN logit is a candidate first
    head2, _ = _rows([0.0, 0.0, 4.0, 0.0, np.nan, 4.0])
    tok, _, _ = rescore.head_rescore(y2, head2, x, 3)
    assert tok == 4                                     # NaN recomputed logit wins
    with pytest.raises(ValueError):
        rescore.head_rescore(y, head, x, 0)
    with pytest.raises(ValueError):
        rescore.head_rescore(y, head, x, 7)


def test_bound_covers_fp32_orders_and_catches_a_dropped_term():
    rng = np.random.default_rng(11)
    K = 3584
    head = (rng.standard_normal((4, K)) * 0.02).astype(np.float16)
    x = (rng.standard_normal(K) * 8).astype(np.float16)
    x[::97] = np.float16(3000.0)                        # large channels, cancellation
    rows = np.arange(4)
    exact = rescore.recompute(head, x, rows)
    bound = rescore.recompute_bound(head, x, rows)
    prods = head.astype(np.float32) * x.astype(np.float32)   # exact in fp32
    seq = np.zeros(4, np.float32)
    for j in range(K):
        seq = seq + prods[:, j]
    pair = prods.copy()
    while pair.shape[1] > 1:
        if pair.shape[1] % 2:
            pair = np.concatenate([pair, np.zeros((4, 1), np.float32)], axis=1)
        pair = pair[:, 0::2] + pair[:, 1::2]
    for got in (seq, pair[:, 0]):
        assert np.all(np.abs(got.astype(np.float64) - exact) <= bound)
    # one dropped product (the largest of each row) is far outside the bound
    j = np.argmax(np.abs(prods), axis=1)
    dropped = exact - prods[rows, j].astype(np.float64)
    assert np.all(np.abs(dropped - exact) > 100 * bound)

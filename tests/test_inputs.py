"""The seeded input generators: shapes, determinism, chunked row sampling."""

import numpy as np

from gemm_tkq_gemv_amd import inputs


def test_shapes_order():
    s = inputs.sweep_shapes("qwen2.5-0.5b")
    assert [n for n, _, _ in s[:7]] == ["L0.q", "L0.k", "L0.v", "L0.o", "L0.gate", "L0.up", "L0.down"]
    assert s[1][1:] == (128, 896) and s[4][1:] == (4864, 896) and s[6][1:] == (896, 4864)
    assert s[-1] == ("lm_head", 151936, 896)
    s7 = inputs.sweep_shapes("qwen2.5-7b")
    assert s7[1][1:] == (512, 3584) and s7[6][1:] == (3584, 18944) and s7[-1][1:] == (152064, 3584)


def test_single_gemv_recipe_deterministic():
    W1, x1 = inputs.single_gemv_896()
    W2, x2 = inputs.single_gemv_896()
    assert W1.dtype == np.float32 and x1.dtype == np.float16
    assert np.array_equal(W1, W2) and np.array_equal(x1, x2)
    assert 0.018 < W1.std() < 0.022


def test_row_sampling_matches_full_matrix():
    W, _ = inputs.sweep_matrix("qwen2.5-0.5b", 4, 4864, 896)
    rows = np.array([4863, 0, 17, 2048, 17])
    got = inputs.sweep_weight_rows("qwen2.5-0.5b", 4, 4864, 896, rows)
    assert np.array_equal(got, W[rows])


def test_binary_case_values():
    W, x = inputs.binary_case(896, 896)
    assert set(np.unique(W).tolist()) == {-1.0, 1.0}
    assert set(np.unique(x).tolist()) == {-1.0, 1.0}

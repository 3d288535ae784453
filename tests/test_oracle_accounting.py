"""Pins of oracle.accounting against the figures the Whetstone page prints.

Golden values: tests/golden/whetstone_roofline.txt (Whetstone, "The one fact
that shapes everything": parameter table and bytes/token table) and
tests/golden/metadata_bits.txt (Whetstone, "What the weights can actually
survive").  Shapes are the Qwen2.5-0.5B linear layers; the page's figures are
reproduced from them by closed form.
"""

import os

import pytest

from gemm_tkq_gemv_amd import inputs
from oracle import accounting as acc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    vals, fmts = {}, {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "fmt":
                fmts[parts[1]] = tuple(float(p) for p in parts[2:])
            else:
                vals[parts[0]] = float(parts[1])
    return vals, fmts


def test_param_table_exact_integers():
    shapes = inputs.sweep_shapes("qwen2.5-0.5b")
    assert len(shapes) == 24 * 7 + 1
    blocks = acc.linear_params(shapes[:-1])
    head = acc.linear_params(shapes[-1:])
    assert blocks == 357_826_560
    assert head == 136_134_656
    assert blocks + head == 493_961_216


def test_param_table_matches_page():
    vals, _ = _read("whetstone_roofline.txt")
    shapes = inputs.sweep_shapes("qwen2.5-0.5b")
    blocks = acc.linear_params(shapes[:-1])
    head = acc.linear_params(shapes[-1:])
    total = blocks + head
    assert round(blocks / 1e6, 1) == vals["params_blocks_M"]
    assert round(head / 1e6, 1) == vals["params_lm_head_M"]
    assert round(total / 1e6, 1) == vals["params_total_M"]
    assert round(100 * blocks / total, 1) == vals["params_blocks_share_pct"]
    assert round(100 * head / total, 1) == vals["params_lm_head_share_pct"]


def test_metadata_bits_per_weight():
    vals, _ = _read("metadata_bits.txt")
    assert acc.meta_bits_per_weight(32, 32) == vals["32"]
    assert acc.meta_bits_per_weight(32, 128) == vals["128"]
    assert acc.bits_per_weight(4, 32, 128) == vals["int4_g128_bpw"]


def test_bytes_per_token_table():
    vals, fmts = _read("whetstone_roofline.txt")
    total = acc.linear_params(inputs.sweep_shapes("qwen2.5-0.5b"))
    bw = vals["bandwidth_GB_s"] * 1e9
    for name, (bpw, mb, ceil) in fmts.items():
        b = acc.bytes_per_token(total, bpw)
        # The page rounds to 0.1 MB; its hier-g32 row uses the format's exact
        # bpw (slightly above the printed 4.28), so allow 0.2 MB there.
        tol_mb = 0.2 if name == "int4_hier_g32" else 0.05 + 1e-9
        assert abs(b / 1e6 - mb) <= tol_mb, name
        # Ceilings are printed as integers; the page's bytes are rounded.
        assert abs(acc.ceiling_tok_s(bw, b) - ceil) <= 1.0, name


def test_ceiling_is_bandwidth_over_bytes():
    # The roofline equation itself: halving bytes doubles the ceiling.
    assert acc.ceiling_tok_s(8e12, 4e9) == 2000.0
    assert acc.ceiling_tok_s(8e12, 2e9) == 4000.0


@pytest.mark.parametrize("fmt,expect", [
    # per-weight stored bytes at K = 896 (no x/y): 0.53125 / 1.015625 / 0.265625 / 0.125
    ("int4", 0.53125), ("k5", 1.015625), ("tern", 0.265625), ("bin", 0.125)])
def test_bytes_per_weight(fmt, expect):
    assert acc.weight_bytes(fmt, 896, 896) / (896 * 896) == expect


def test_sweep_bytes_int4():
    shapes = inputs.sweep_shapes("qwen2.5-0.5b")
    w = sum(acc.weight_bytes("int4", n, k) for _, n, k in shapes)
    assert w == 262_416_896
    # weights + meta, plus every x (fp16) and y (fp16) once
    assert acc.sweep_bytes("int4", shapes) == 262_416_896 + 493_312 + 912_128
    # 4.25 bits/weight exactly
    total = acc.linear_params(shapes)
    assert w * 8 == int(4.25 * total)


def test_sweep_bytes_other_codings():
    shapes = inputs.sweep_shapes("qwen2.5-0.5b")
    assert sum(acc.weight_bytes("k5", n, k) for _, n, k in shapes) == 501_679_360
    assert sum(acc.weight_bytes("tern", n, k) for _, n, k in shapes) == 131_208_448
    s7 = inputs.sweep_shapes("qwen2.5-7b")
    assert len(s7) == 28 * 7 + 1
    assert sum(acc.weight_bytes("int4", n, k) for _, n, k in s7) == 3_756_089_344


def test_prefill_flops():
    tot = sum(acc.gemm_flops(512, n, k) for _, n, k in inputs.prefill_shapes())
    assert tot == 208_574_349_312


def test_int2_bytes_match_page_row():
    # Whetstone bytes/token table: int2 g128 at 2.25 bits/weight, 138.9 MB
    vals, fmts = _read("whetstone_roofline.txt")
    shapes = inputs.sweep_shapes("qwen2.5-0.5b")
    total = sum(acc.weight_bytes("int2", n, k) for _, n, k in shapes)
    bpw, mb, _ = fmts["int2_g128"]
    assert 8.0 * total / acc.linear_params(shapes) == bpw
    assert abs(total / 1e6 - mb) <= 0.05 + 1e-9


def test_int3_bytes_match_page_row():
    # Whetstone bytes/token table: int3 g128 at 3.25 bits/weight, 200.7 MB
    vals, fmts = _read("whetstone_roofline.txt")
    shapes = inputs.sweep_shapes("qwen2.5-0.5b")
    total = sum(acc.weight_bytes("int3", n, k) for _, n, k in shapes)
    bpw, mb, _ = fmts["int3_g128"]
    assert 8.0 * total / acc.linear_params(shapes) == bpw
    assert abs(total / 1e6 - mb) <= 0.05 + 1e-9

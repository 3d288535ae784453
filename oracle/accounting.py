"""Byte and roofline accounting (test infrastructure only).

Whetstone, "The one fact that shapes everything":
  * the roofline equation: ceiling (tok/s) = bandwidth / bytes per token;
  * the parameter table: transformer blocks vs the tied lm_head, both read on
    every token;
  * the bytes/token table: bytes = params * bits_per_weight / 8 per format.
Whetstone, "What the weights can actually survive": per-group metadata of one
fp16 scale and one fp16 zero-point amounts to 32/G bits per weight for groups
of G weights.

Shapes are passed in as (name, N, K) tuples; nothing here knows a model.
"""


def linear_params(shapes):
    """Number of weights of a list of (name, N, K) linear layers."""
    return sum(int(n) * int(k) for _, n, k in shapes)


def meta_bits_per_weight(meta_bits_per_group, group):
    """Metadata cost: e.g. fp16 scale + fp16 zero (32 bits) per 128 -> 0.25."""
    return meta_bits_per_group / group


def bits_per_weight(code_bits, meta_bits_per_group, group):
    return code_bits + meta_bits_per_weight(meta_bits_per_group, group)


def bytes_per_token(params, bpw):
    """Weight bytes read per decoded token: params * bits/weight / 8."""
    return params * bpw / 8.0


def ceiling_tok_s(bandwidth_bytes_s, bytes_token):
    """The roofline: ceiling (tok/s) = bandwidth / bytes per token."""
    return bandwidth_bytes_s / bytes_token


# Exact stored bytes of one GEMV for each coding: packed codes + per-group
# metadata + the x vector read once + the y vector written once.
#   int4 g128 : K/2 code bytes + 4 bytes (fp16 scale, fp16 zero) per 128
#   K5        : K code bytes   + 2 bytes (fp16 scale) per 128
#   ternary   : K/4 code bytes + 2 bytes (fp16 scale) per 128
#   binary    : K/8 code bytes, no metadata, x is K/8 bytes, y is int32
#   int3 g128 : 3K/8 code bytes + 4 bytes (fp16 scale, fp16 zero) per 128
#   int2 g128 : K/4 code bytes + 4 bytes (fp16 scale, fp16 zero) per 128
#   int4-hier-g32: K/2 code bytes + 1 byte (two 4-bit indices) per 32
#               + 4 bytes (fp16 pair) per row
_FMT_BYTES = {
    "int3": (lambda n, k: n * (3 * k // 8) + n * (k // 128) * 4, lambda k: 2 * k, lambda n: 2 * n),
    "int2": (lambda n, k: n * (k // 4) + n * (k // 128) * 4, lambda k: 2 * k, lambda n: 2 * n),
    "hier": (lambda n, k: n * (k // 2) + n * (k // 32) + 4 * n, lambda k: 2 * k, lambda n: 2 * n),
    "int4": (lambda n, k: n * (k // 2) + n * (k // 128) * 4, lambda k: 2 * k, lambda n: 2 * n),
    "k5": (lambda n, k: n * k + n * (k // 128) * 2, lambda k: 2 * k, lambda n: 2 * n),
    "tern": (lambda n, k: n * (k // 4) + n * (k // 128) * 2, lambda k: 2 * k, lambda n: 2 * n),
    "bin": (lambda n, k: n * (k // 8), lambda k: k // 8, lambda n: 4 * n),
}


def weight_bytes(fmt, N, K):
    """Packed codes + metadata bytes of one N x K matrix."""
    return _FMT_BYTES[fmt][0](int(N), int(K))


def gemv_bytes(fmt, N, K):
    """Algorithmic bytes of one GEMV: weights + meta + x + y, each once."""
    w, xb, yb = _FMT_BYTES[fmt]
    return w(int(N), int(K)) + xb(int(K)) + yb(int(N))


def sweep_bytes(fmt, shapes):
    """Algorithmic bytes of one decode-equivalent sweep over all matrices."""
    return sum(gemv_bytes(fmt, n, k) for _, n, k in shapes)


def gemm_flops(M, N, K):
    """2*M*N*K multiply-add flops of Y = X . W^T."""
    return 2 * int(M) * int(N) * int(K)


def gemm_bytes(fmt, M, N, K):
    """Algorithmic bytes of the prefill GEMM: packed W + meta once, X (fp16)
    once, Y (fp16) once."""
    return weight_bytes(fmt, N, K) + 2 * int(M) * int(K) + 2 * int(M) * int(N)

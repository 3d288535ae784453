"""Packers and unpackers for the four code layouts (test infrastructure only).

Layouts (the library's storage contract; Whetstone, "The .wstone format"
fixes the nibble order only as the one the GEMV's 16-byte loads read; the
reading taken here is the natural little-endian order, which a 16-byte load
of a row reads front to back):

* int4 codes   uint32 [N][K/8]: element 8j+i of a row in bits [4i, 4i+4) of
                word j.
* int4 meta    uint32 [N][K/128]: fp16 scale bits in bits [0,16), fp16 zero
                bits in bits [16,32) (a little-endian half2 {scale, zero}).
* K5 codes     uint8 [N][K] (one byte per weight), fp16 scale [N][K/128].
* ternary      uint32 [N][K/16]: element 16j+i in bits [2i, 2i+2) of word j,
                code = t + 1; fp16 scale [N][K/128].
* binary       uint32 [N][K/32]: element 32j+i in bit i of word j.
* int2         uint32 [N][K/16]: element 16j+i in bits [2i, 2i+2) of word j
                (the ternary field layout), meta as int4 (half2 {scale, zero}).
* int3         3 bits per weight, 3*N*K/8 bytes, meta as int4.  The
                pages fix only the density (3.25 bits/weight with the g128
                metadata); the layout is chosen for the GEMV's 16-byte loads:
                within a 128-group, block b (codes 32b..32b+31) is three
                32-bit words W0, W1, W2; word Wj holds code 10j+f in bits
                [3f, 3f+3) and code 10j+5+f in bits [16+3f, 16+3f+3) for
                f = 0..4, and bit j of code 30 in bit 15, bit j of code 31 in
                bit 31.  The group's 12 words (b0W0, b0W1, b0W2, b1W0, ...)
                form three 16-byte planes (words 0-3, 4-7, 8-11).  The matrix
                is stored plane-major, uint32 [3][N][K/32]: plane p of group g
                of row n sits at byte p*N*K/8 + n*K/8 + 16*g, so each plane of
                consecutive rows is one contiguous run.
* int4-hier-g32 codes as int4; one metadata block per matrix:
                bytes [0, N*K/32): byte n*(K/32)+g = sc | (mi << 4) of group g
                of row n; zero padding up to a multiple of 16 bytes (offset
                R); then uint32 [N] at R: fp16 d in bits [0,16), fp16 dmin in
                bits [16,32).

Packers build words by multiply-and-add over slots; unpackers read a slot with
shift-and-mask.  They are written independently from the layout text above.
"""

import numpy as np


def _pack_fields(codes, bits):
    codes = np.asarray(codes)
    if codes.ndim != 2:
        raise ValueError("codes must be 2-D")
    per = 32 // bits
    N, K = codes.shape
    if K % per:
        raise ValueError("K must be a multiple of %d" % per)
    c = codes.astype(np.uint64).reshape(N, K // per, per)
    if np.any(c >> np.uint64(bits)):
        raise ValueError("code does not fit in %d bits" % bits)
    weights = (np.uint64(1) << (np.uint64(bits) * np.arange(per, dtype=np.uint64)))
    return (c * weights).sum(axis=2).astype(np.uint32)


def _unpack_fields(words, K, bits):
    words = np.asarray(words, dtype=np.uint32)
    per = 32 // bits
    N = words.shape[0]
    out = np.empty((N, K), dtype=np.uint8)
    mask = np.uint32((1 << bits) - 1)
    for i in range(per):
        out[:, i::per] = ((words[:, : K // per] >> np.uint32(bits * i)) & mask).astype(np.uint8)
    return out


def pack_int4(q):
    """int4 codes [N,K] (0..15) -> uint32 [N,K/8], LSB-first nibbles."""
    return _pack_fields(q, 4)


def unpack_int4(words, K):
    """uint32 [N,K/8] -> int4 codes uint8 [N,K]."""
    return _unpack_fields(words, K, 4)


def pack_int4_meta(scale16, zero16):
    """fp16 scale and fp16 zero [N,K/128] -> uint32 half2 {scale lo, zero hi}."""
    s = np.asarray(scale16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    z = np.asarray(zero16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    return s + z * np.uint32(65536)


def unpack_int4_meta(meta):
    """uint32 half2 [N,K/128] -> (scale fp16, zero fp16)."""
    meta = np.asarray(meta, dtype=np.uint32)
    s = (meta & np.uint32(0xFFFF)).astype(np.uint16).view(np.float16)
    z = (meta >> np.uint32(16)).astype(np.uint16).view(np.float16)
    return s, z


def pack_tern(codes):
    """ternary codes [N,K] (0..2) -> uint32 [N,K/16], LSB-first 2-bit fields."""
    return _pack_fields(codes, 2)


def unpack_tern(words, K):
    return _unpack_fields(words, K, 2)


def _int3_block_words(c):
    """32 codes (uint64 array [..., 32]) -> the block's 3 words [..., 3]."""
    words = []
    for j in range(3):
        w = np.zeros(c.shape[:-1], dtype=np.uint64)
        for f in range(5):
            w = w + c[..., 10 * j + f] * np.uint64(1 << (3 * f))
            w = w + c[..., 10 * j + 5 + f] * np.uint64(1 << (16 + 3 * f))
        w = w + ((c[..., 30] >> np.uint64(j)) & np.uint64(1)) * np.uint64(1 << 15)
        w = w + ((c[..., 31] >> np.uint64(j)) & np.uint64(1)) * np.uint64(1 << 31)
        words.append(w)
    return np.stack(words, axis=-1)


def pack_int3(q):
    """int3 codes [N,K] (0..7) -> uint32 [3, N, K/32] in the plane-major layout."""
    q = np.asarray(q)
    N, K = q.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    c = q.astype(np.uint64)
    if np.any(c > 7):
        raise ValueError("code does not fit in 3 bits")
    ng = K // 128
    blocks = c.reshape(N, ng, 4, 32)
    words = _int3_block_words(blocks).reshape(N, ng, 12)          # b0W0 b0W1 b0W2 b1W0 ...
    planes = words.reshape(N, ng, 3, 4).transpose(2, 0, 1, 3)      # [plane][N][group][4]
    return planes.reshape(3, N, ng * 4).astype(np.uint32)


def unpack_int3(words, K):
    """uint32 [3, N, K/32] -> int3 codes uint8 [N,K] (shift-and-mask reads)."""
    words = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    ng = K // 128
    N = words.size // (3 * ng * 4)
    w = words.reshape(3, N, ng, 4).transpose(1, 2, 0, 3).reshape(N, ng, 4, 3)
    out = np.zeros((N, ng, 4, 32), dtype=np.uint8)
    for j in range(3):
        wj = w[..., j]
        for f in range(5):
            out[..., 10 * j + f] = (wj >> np.uint64(3 * f)) & np.uint64(7)
            out[..., 10 * j + 5 + f] = (wj >> np.uint64(16 + 3 * f)) & np.uint64(7)
        out[..., 30] |= (((wj >> np.uint64(15)) & np.uint64(1)) << np.uint64(j)).astype(np.uint8)
        out[..., 31] |= (((wj >> np.uint64(31)) & np.uint64(1)) << np.uint64(j)).astype(np.uint8)
    return out.reshape(N, K)


def pack_int2(q):
    """int2 codes [N,K] (0..3) -> uint32 [N,K/16], LSB-first 2-bit fields."""
    return _pack_fields(q, 2)


def unpack_int2(words, K):
    return _unpack_fields(words, K, 2)


def pack_bits(bits):
    """sign bits [N,K] (0/1) -> uint32 [N,K/32], bit i of word j = element 32j+i."""
    return _pack_fields(bits, 1)


def unpack_bits(words, K):
    return _unpack_fields(words, K, 1)


def hier_row_offset(N, K):
    """Byte offset R of the per-row fp16 pairs in an int4-hier-g32 metadata
    block: the group bytes rounded up to a multiple of 16."""
    gb = int(N) * (int(K) // 32)
    return (gb + 15) // 16 * 16


def hier_meta_bytes(N, K):
    """Size of an int4-hier-g32 metadata block."""
    return hier_row_offset(N, K) + 4 * int(N)


def pack_hier_meta(sc, mi, d16, dmin16):
    """(sc, mi uint8 [N,K/32] in 0..15; d16, dmin16 fp16 [N]) -> uint8 block."""
    sc = np.asarray(sc, dtype=np.uint8)
    mi = np.asarray(mi, dtype=np.uint8)
    if np.any(sc > 15) or np.any(mi > 15):
        raise ValueError("index does not fit in 4 bits")
    N, ng = sc.shape
    K = ng * 32
    out = np.zeros(hier_meta_bytes(N, K), dtype=np.uint8)
    out[: N * ng] = (sc.astype(np.uint32) + mi.astype(np.uint32) * 16).reshape(-1).astype(np.uint8)
    R = hier_row_offset(N, K)
    rows = pack_int4_meta(np.asarray(d16, dtype=np.float16).reshape(N, 1),
                          np.asarray(dmin16, dtype=np.float16).reshape(N, 1)).reshape(N)
    out[R:R + 4 * N] = rows.astype("<u4").view(np.uint8)
    return out


def unpack_hier_meta(block, N, K):
    """uint8 block -> (sc uint8 [N,K/32], mi uint8 [N,K/32], d16 fp16 [N],
    dmin16 fp16 [N])."""
    block = np.asarray(block, dtype=np.uint8)
    ng = int(K) // 32
    g = block[: N * ng].reshape(N, ng)
    R = hier_row_offset(N, K)
    rows = block[R:R + 4 * N].copy().view("<u4")
    d16, dmin16 = unpack_int4_meta(rows)
    return g & np.uint8(15), g >> np.uint8(4), d16, dmin16

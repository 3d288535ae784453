"""Round-to-nearest quantizers of the oracle (test infrastructure only).

All arithmetic is IEEE fp32 in numpy, step by step, so that an fp32 GPU
quantizer executing the same operations produces bit-identical codes and
fp16 metadata.  Rounding is ``rint`` (round half to even); fp32 -> fp16 is
the IEEE round-to-nearest-even conversion; division is true fp32 division.

The pages never print a quantizer's formulas.  What they fix, and the reading
taken where they are silent:

* Whetstone, "What the weights can actually survive" (quality table and the
  quantizer table): the group-128 int4 format is round-to-nearest with a
  group size of 128, with one fp16 scale and one fp16 zero-point for every
  128 weights (32 metadata bits per group, 0.25 bits/weight).  Reading: asymmetric min/max RTN over the
  group's range widened to include 0, ``w ~ s * (q - z)``, q in 0..15, z an
  integer zero-point stored in fp16.
* Whetstone, status list: a shared fp16 scale underflowing to zero packed
  rows as garbage.  Reading: a scale that rounds to fp16 zero is replaced by
  1.0 (the group is then all zero-point codes and dequantizes to 0).
* TKintegers K5, "What is K5?": one byte per weight, five balanced trits, 243
  values.  Reading: symmetric absmax RTN onto the integers -121..121 with an
  fp16 scale per 128 weights; the byte is the value plus 121.
* Whetstone, bytes/token table and quality table ("ternary g128"): ternary
  with group 128, round-to-nearest.  Reading: scale = mean |w| of the group
  (absmean), summed sequentially in k order in fp32; t = clip(rint(w/s),
  -1, 1); stored code t + 1.
* Whetstone, "Measured hardware facts": {-1,+1} values packed as bits {1,0}.
  Reading: bit = 1 exactly when the value is negative.
* Whetstone, bytes/token table ("int4 hier-g32", 4.28 bits/weight), the
  quantizer table ("group 32 with hierarchical scale metadata") and "Prior
  art" (the Q4_K comparison): int4 in groups of 32 whose scale and offset are
  4-bit indices against one fp16 pair per row.  Reading, as in Q4_K: each
  group has a scale index sc and a min index mi, the row has fp16 (d, dmin),
  and w ~ d*sc*q - dmin*mi with q in 0..15; RTN at every level (the pages
  print no fitting procedure).
"""

import numpy as np

F32 = np.float32
GROUP = 128


def fp16_rne(a):
    """fp32 -> fp16 with IEEE round-to-nearest-even (numpy's conversion)."""
    return np.asarray(a, dtype=np.float32).astype(np.float16)


def _guard_zero_scale(s16):
    """Replace an fp16 scale that rounded to zero by 1.0.

    Whetstone, status list (the 7B underflow bug): a zero scale must never be
    stored.  With scale 1.0 every weight of such a group rounds to the
    zero-point code, so the group dequantizes to exactly 0.
    """
    s16 = np.array(s16, dtype=np.float16, copy=True)
    s16[s16 == 0] = np.float16(1.0)
    return s16


def _groups(W):
    W = np.asarray(W, dtype=np.float32)
    if W.ndim != 2 or W.shape[1] % GROUP:
        raise ValueError("W must be [N, K] with K a multiple of 128")
    N, K = W.shape
    return W.reshape(N, K // GROUP, GROUP)


def quantize_int4_g128(W):
    """int4, group 128, asymmetric round-to-nearest (Whetstone, "What the
    weights can actually survive": RTN group-128 format, f16 scale + f16 zero).

    Per row n and group g, in fp32:
      lo = min(min_k w, 0); hi = max(max_k w, 0)
      s  = (hi - lo) / 15            (true division)
      s16 = fp16_rne(s); s16 := 1 if s16 == 0
      z  = clip(rint(-lo / s16), 0, 15)            (integer, stored as fp16)
      q  = clip(rint(w / s16) + z, 0, 15)

    Returns (q uint8 [N,K], scale fp16 [N,K/128], zero fp16 [N,K/128]).
    """
    G = _groups(W)
    N, ng, _ = G.shape
    lo = np.minimum(G.min(axis=2), F32(0))
    hi = np.maximum(G.max(axis=2), F32(0))
    s = (hi - lo) / F32(15)
    s16 = _guard_zero_scale(fp16_rne(s))
    sf = s16.astype(np.float32)
    z = np.clip(np.rint(-lo / sf), F32(0), F32(15)).astype(np.int32)
    q = np.rint(G / sf[:, :, None]) + z[:, :, None].astype(np.float32)
    q = np.clip(q, F32(0), F32(15)).astype(np.uint8)
    return q.reshape(N, ng * GROUP), s16, z.astype(np.float16)


def quantize_int2_g128(W):
    """int2, group 128, asymmetric round-to-nearest (Whetstone, bytes/token
    table and quality table: "int2 g128" at 2.25 bits/weight = 2-bit codes
    plus the same 32 metadata bits per 128 as int4 g128).  Reading: the int4
    g128 quantizer with four levels.

    Per row n and group g, in fp32:
      lo = min(min_k w, 0); hi = max(max_k w, 0)
      s  = (hi - lo) / 3;  s16 = fp16_rne(s); s16 := 1 if s16 == 0
      z  = clip(rint(-lo / s16), 0, 3)             (integer, stored as fp16)
      q  = clip(rint(w / s16) + z, 0, 3)

    Returns (q uint8 [N,K], scale fp16 [N,K/128], zero fp16 [N,K/128]).
    """
    G = _groups(W)
    N, ng, _ = G.shape
    lo = np.minimum(G.min(axis=2), F32(0))
    hi = np.maximum(G.max(axis=2), F32(0))
    s16 = _guard_zero_scale(fp16_rne((hi - lo) / F32(3)))
    sf = s16.astype(np.float32)
    z = np.clip(np.rint(-lo / sf), F32(0), F32(3)).astype(np.int32)
    q = np.rint(G / sf[:, :, None]) + z[:, :, None].astype(np.float32)
    q = np.clip(q, F32(0), F32(3)).astype(np.uint8)
    return q.reshape(N, ng * GROUP), s16, z.astype(np.float16)


def quantize_int3_g128(W):
    """int3, group 128, asymmetric round-to-nearest (Whetstone, bytes/token
    and quality tables: "int3 g128" at 3.25 bits/weight = 3-bit codes plus
    the same 32 metadata bits per 128 as int4 g128).  Reading: the int4 g128
    quantizer with eight levels.

    Per row n and group g, in fp32:
      lo = min(min_k w, 0); hi = max(max_k w, 0)
      s  = (hi - lo) / 7;  s16 = fp16_rne(s); s16 := 1 if s16 == 0
      z  = clip(rint(-lo / s16), 0, 7)             (integer, stored as fp16)
      q  = clip(rint(w / s16) + z, 0, 7)

    Returns (q uint8 [N,K], scale fp16 [N,K/128], zero fp16 [N,K/128]).
    """
    G = _groups(W)
    N, ng, _ = G.shape
    lo = np.minimum(G.min(axis=2), F32(0))
    hi = np.maximum(G.max(axis=2), F32(0))
    s16 = _guard_zero_scale(fp16_rne((hi - lo) / F32(7)))
    sf = s16.astype(np.float32)
    z = np.clip(np.rint(-lo / sf), F32(0), F32(7)).astype(np.int32)
    q = np.rint(G / sf[:, :, None]) + z[:, :, None].astype(np.float32)
    q = np.clip(q, F32(0), F32(7)).astype(np.uint8)
    return q.reshape(N, ng * GROUP), s16, z.astype(np.float16)


def quantize_k5(W):
    """K5 byte codes, fp16 scale per 128 weights (TKintegers K5, "What is K5?").

    Per row n and group g, in fp32:
      a   = max_k |w|
      s16 = fp16_rne(a / 121); s16 := 1 if s16 == 0
      v   = clip(rint(w / s16), -121, 121)
      c   = v + 121         (uint8, 0..242)

    Returns (c uint8 [N,K], scale fp16 [N,K/128]).
    """
    G = _groups(W)
    N, ng, _ = G.shape
    a = np.abs(G).max(axis=2)
    s16 = _guard_zero_scale(fp16_rne(a / F32(121)))
    sf = s16.astype(np.float32)
    v = np.clip(np.rint(G / sf[:, :, None]), F32(-121), F32(121))
    c = (v.astype(np.int32) + 121).astype(np.uint8)
    return c.reshape(N, ng * GROUP), s16


def absmean_sequential(G):
    """fp32 mean of |w| over the last axis, summed strictly in k order.

    ``np.add.accumulate`` is an element-by-element running sum, so its last
    element is ((|w0| + |w1|) + |w2|) + ... in fp32.  Division by 128 is exact.
    """
    a = np.abs(np.asarray(G, dtype=np.float32))
    total = np.add.accumulate(a, axis=-1, dtype=np.float32)[..., -1]
    return total / F32(GROUP)


def quantize_tern_g128(W):
    """Ternary g128 (Whetstone, bytes/token and quality tables, "ternary g128",
    round-to-nearest).

    Per row n and group g, in fp32:
      m   = (sequential k-order sum of |w|) / 128
      s16 = fp16_rne(m); s16 := 1 if s16 == 0
      t   = clip(rint(w / s16), -1, 1)
      code = t + 1          (0, 1, 2)

    Returns (code uint8 [N,K], scale fp16 [N,K/128]).
    """
    G = _groups(W)
    N, ng, _ = G.shape
    s16 = _guard_zero_scale(fp16_rne(absmean_sequential(G)))
    sf = s16.astype(np.float32)
    t = np.clip(np.rint(G / sf[:, :, None]), F32(-1), F32(1))
    code = (t.astype(np.int32) + 1).astype(np.uint8)
    return code.reshape(N, ng * GROUP), s16


def sign_bits(W):
    """Binary sign code (Whetstone, "Measured hardware facts": {-1,+1} packed as
    bits {1,0}).  bit = 1 exactly when w < 0; -0.0 and +values give 0."""
    return (np.asarray(W, dtype=np.float32) < 0).astype(np.uint8)


HIER_GROUP = 32


def quantize_int4_hier_g32(W):
    """int4 with group 32 and two-level scales (Whetstone, quantizer table:
    "group 32 with hierarchical scale metadata"; "Prior art": like Q4_K's
    sub-scales against a super-block fp16 pair, but the super-block is a whole
    row and the indices have 4 bits).

    Per row n, in fp32 (every division true division, every rint half-even):
      per group g of 32:  lo = min(min_k w, 0); hi = max(max_k w, 0)
                          s_g = (hi - lo) / 15      (wanted step)
                          m_g = -lo                 (wanted offset, >= 0)
      d16    = fp16_rne(max_g s_g / 15);  d16 := 1 if d16 == 0
      dmin16 = fp16_rne(max_g m_g / 15);  dmin16 := 1 if dmin16 == 0
               (Whetstone, status list: a shared fp16 row scale that
               underflows to zero must not be stored)
      sc_g = clip(rint(s_g / d16), 1, 15)     (never 0: a group keeps a step)
      mi_g = clip(rint(m_g / dmin16), 0, 15)
      step_g = d16 * sc_g;  off_g = dmin16 * mi_g    (exact in fp32)
      q = clip(rint((w + off_g) / step_g), 0, 15)

    Dequantized weight: d16 * sc_g * q - dmin16 * mi_g.

    Returns (q uint8 [N,K], sc uint8 [N,K/32], mi uint8 [N,K/32],
             d16 fp16 [N], dmin16 fp16 [N]).
    """
    W = np.asarray(W, dtype=np.float32)
    if W.ndim != 2 or W.shape[1] % HIER_GROUP:
        raise ValueError("W must be [N, K] with K a multiple of 32")
    N, K = W.shape
    G = W.reshape(N, K // HIER_GROUP, HIER_GROUP)
    lo = np.minimum(G.min(axis=2), F32(0))
    hi = np.maximum(G.max(axis=2), F32(0))
    s = (hi - lo) / F32(15)
    m = -lo
    d16 = _guard_zero_scale(fp16_rne(s.max(axis=1) / F32(15)))
    dmin16 = _guard_zero_scale(fp16_rne(m.max(axis=1) / F32(15)))
    df = d16.astype(np.float32)[:, None]
    mf = dmin16.astype(np.float32)[:, None]
    sc = np.clip(np.rint(s / df), F32(1), F32(15))
    mi = np.clip(np.rint(m / mf), F32(0), F32(15))
    step = df * sc
    off = mf * mi
    q = np.clip(np.rint((G + off[:, :, None]) / step[:, :, None]), F32(0), F32(15))
    return (q.astype(np.uint8).reshape(N, K), sc.astype(np.uint8), mi.astype(np.uint8),
            d16, dmin16)

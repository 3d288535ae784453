"""CPU oracle for the low-bit weight GEMV path.  TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously-correct reference that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product package
(``gemm_tkq_gemv_amd``) never imports it, and this package imports nothing from
the product package: the two share no code.  Seeded inputs are generated
elsewhere and passed in as plain numpy arrays.

Contents
--------
quant       round-to-nearest quantizers: int4 g128 (asymmetric, fp16 scale and
            zero), K5 balanced-ternary byte codes, ternary g128 (absmean),
            binary sign bits.
pack        packers and unpackers for the four code layouts.
ref         dequantization and the fp64 GEMV / GEMM definitions, the per-row
            tolerance bound, and the XOR-popcount binary GEMV.
accounting  parameter counts, bits/weight, bytes per token and the
            bandwidth / bytes roofline ceiling.
kv          the paged 4-bit KV cache (K per channel, V per token, pages of
            128 tokens) and single-query decode attention in fp64, with its
            derived tolerance.
rescore     greedy selection with head rescore: the k largest stored logits
            as candidates, their logits recomputed exactly from the fp16
            output projection, the largest recomputed one as the token.

Every function cites the page passage it follows.  Pages are cited by title
and section: "Whetstone" (the Whetstone README), "TKintegers K5" (the
TKintegers K5 news digest) and "BitDecoding" (the BitDecoding README).

Pins: each function is checked by the ``-m "not gpu"`` tests against values
the pages print, closed forms, exhaustive enumeration on tiny inputs, or
invariants.  Parity status per function is listed in ``tests/test_oracle_*``.
There is no "parity unpinned" function in this package: the float GEMV/GEMM
reduce to the plain definition ``y = W_deq . x`` in fp64 and are pinned by
closed-form special cases and brute force on tiny inputs.
"""

from . import accounting, pack, quant, ref, rescore  # noqa: F401

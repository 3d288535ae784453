"""MI355X-native low-bit weight GEMV (y = dequant(W_q) . x) and its prefill GEMM.

The compute path is the C-ABI library ``libtkq.so`` (hand-written HIP for
gfx950, declared in ``include/tkq.h``); :mod:`gemm_tkq_gemv_amd.tkq` is a thin
ctypes binding with the same entry-point names.  :mod:`.inputs` generates the
seeded synthetic workloads.  Importing this package loads nothing; the
library is loaded on first use of :mod:`.tkq`.
"""

__version__ = "0.1.0"

"""ctypes binding of libtkq (include/tkq.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  The raw
C entry points are exposed under their C names through :func:`lib`; the
functions below take torch tensors, allocate outputs with torch, and call the
entry point of the same name.

Storage dtypes: packed 32-bit words are held in ``torch.int32`` tensors (the
bits are the uint32 words of the layout), fp16 scales in ``torch.float16``.

If ``libtkq.so`` has not been built this module raises on first use; there is
no fallback path.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtkq.so")

FMT_INT4_G128 = 1
FMT_K5_G128 = 2
FMT_TERN_G128 = 3
FMT_BIN = 4
FMT_INT4_HIER_G32 = 5
FMT_INT2_G128 = 6
FMT_INT3_G128 = 7
FORMATS = {"int4": FMT_INT4_G128, "k5": FMT_K5_G128, "tern": FMT_TERN_G128, "bin": FMT_BIN,
           "hier": FMT_INT4_HIER_G32, "int2": FMT_INT2_G128, "int3": FMT_INT3_G128}

OK, EINVAL, ESHAPE, EALIGN, EFORMAT, EHIP, EPLAN = 0, -1, -2, -3, -4, -5, -6


class TkqError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        msg = "%s failed: %s (status %d)" % (what, strerror(status), status)
        if status == EHIP:
            msg += ", hipError_t %d" % lib().tkq_last_hip_error()
        super().__init__(msg)


class GemvDesc(ctypes.Structure):
    """tkq_gemv_desc (64 bytes)."""
    _fields_ = [("fmt", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("work0", ctypes.c_int32), ("big_tiles", ctypes.c_int32),
                ("rows_per_tile", ctypes.c_int32), ("shape", ctypes.c_int32),
                ("small_rows", ctypes.c_int32), ("codes", ctypes.c_void_p),
                ("meta", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class GemvPlan(ctypes.Structure):
    """tkq_gemv_plan (32 bytes)."""
    _fields_ = [("fmt", ctypes.c_int32), ("count", ctypes.c_int32), ("tiles", ctypes.c_int64),
                ("variant", ctypes.c_int32), ("magic", ctypes.c_int32),
                ("reserved", ctypes.c_int64)]


_I64, _I32, _P = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
_SIGNATURES = {
    "tkq_version": ([], ctypes.c_int),
    "tkq_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "tkq_last_hip_error": ([], ctypes.c_int),
    "tkq_pack_int4_g128": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "tkq_pack_k5": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "tkq_pack_tern_g128": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "tkq_pack_bin": ([_P, _I64, _I64, _P, _P], ctypes.c_int),
    "tkq_pack_int4_hier_g32": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "tkq_pack_int2_g128": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "tkq_pack_int3_g128": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "tkq_hier_meta_bytes": ([_I64, _I64], ctypes.c_int64),
    "tkq_gemv_prepare": ([ctypes.POINTER(GemvDesc), _I32, ctypes.POINTER(GemvPlan)], ctypes.c_int),
    "tkq_gemv": ([ctypes.POINTER(GemvPlan), _P, _P], ctypes.c_int),
    "tkq_gemv_argmax": ([ctypes.POINTER(GemvPlan), _P, _I32, _P, _P, _I64, _P], ctypes.c_int),
    "tkq_gemv_argmax_static": ([ctypes.POINTER(GemvPlan), _P, _I32, _P, _P], ctypes.c_int),
    "tkq_gemm_small_prepare": ([ctypes.POINTER(GemvDesc), _I32, _I32, ctypes.POINTER(GemvPlan)],
                               ctypes.c_int),
    "tkq_gemm_small": ([ctypes.POINTER(GemvPlan), _P, _P], ctypes.c_int),
    "tkq_kv_cache_bytes": ([_I32, _I32, _I32], ctypes.c_int64),
    "tkq_kv_decode_workspace_bytes": ([_I32, _I32, _I32, _I32], ctypes.c_int64),
    "tkq_kv_pack": ([_P, _P, _I32, _I32, _I32, _I32, _P, _P], ctypes.c_int),
    "tkq_kv_pack_varlen": ([_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P], ctypes.c_int),
    "tkq_kv_decode": ([_P, _P, _I32, _I32, _I32, _I32, _I32, ctypes.c_float, _P, _P, _I64, _P], ctypes.c_int),
    "tkq_kv_decode_varlen": ([_P, _P, _P, _I32, _I32, _I32, _I32, _I32, ctypes.c_float, _P, _P, _I64, _P],
                             ctypes.c_int),
    "tkq_gemm_prefill": ([_I32, _I64, _I64, _I64, _P, _P, _P, _P, _P, _I64, _P], ctypes.c_int),
    "tkq_read_probe": ([_P, _I64, _P, _P], ctypes.c_int),
    "tkq_head_rescore": ([_P, _I64, _P, _P, _I64, _I32, _P, _P, _P, _P], ctypes.c_int),
    "tkq_gemv_argmax_rescore": ([ctypes.POINTER(GemvPlan), _P, _I32, _I64, _I64, _P, _I32, _P, _P, _P, _P, _I64,
                                 _P], ctypes.c_int),
}

_lib = None


def lib():
    """The loaded libtkq.so with argument types set (raises if not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtkq.so is not built (python -m gemm_tkq_gemv_amd.build); "
                               "there is no fallback path")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def strerror(status):
    return lib().tkq_strerror(status).decode()


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != OK:
        raise TkqError(st, name)


def _stream(stream=None, *owned):
    """The stream to enqueue on (the current one by default), as a void*.

    Tensors this binding allocated (on the current stream) and hands to a
    kernel on another stream are marked as used by that stream, so that the
    caching allocator does not give their memory to a new allocation before
    that stream's work is done."""
    cur = torch.cuda.current_stream()
    s = stream if stream is not None else cur
    if stream is not None and stream != cur:
        for t in owned:
            if t is not None:
                t.record_stream(stream)
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, name, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t


# ---- quantize + pack ---------------------------------------------------------

def pack_int4_g128(W, stream=None):
    """W fp32 [N,K] -> (codes int32 [N,K/8], meta int32 [N,K/128] = half2 {s,z})."""
    _need(W, torch.float32, "W")
    N, K = W.shape
    codes = torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    meta = torch.empty((N, K // 128), dtype=torch.int32, device=W.device)
    _call("tkq_pack_int4_g128", _ptr(W), N, K, _ptr(codes), _ptr(meta), _stream(stream, codes, meta))
    return codes, meta


def pack_k5(W, stream=None):
    """W fp32 [N,K] -> (codes uint8 [N,K], scale fp16 [N,K/128])."""
    _need(W, torch.float32, "W")
    N, K = W.shape
    codes = torch.empty((N, K), dtype=torch.uint8, device=W.device)
    scale = torch.empty((N, K // 128), dtype=torch.float16, device=W.device)
    _call("tkq_pack_k5", _ptr(W), N, K, _ptr(codes), _ptr(scale), _stream(stream, codes, scale))
    return codes, scale


def pack_tern_g128(W, stream=None):
    """W fp32 [N,K] -> (codes int32 [N,K/16], scale fp16 [N,K/128])."""
    _need(W, torch.float32, "W")
    N, K = W.shape
    codes = torch.empty((N, K // 16), dtype=torch.int32, device=W.device)
    scale = torch.empty((N, K // 128), dtype=torch.float16, device=W.device)
    _call("tkq_pack_tern_g128", _ptr(W), N, K, _ptr(codes), _ptr(scale), _stream(stream, codes, scale))
    return codes, scale


def pack_bin(W, stream=None):
    """W fp32 [N,K] (or [K]) -> sign bits int32 [N,K/32] (or [K/32])."""
    _need(W, torch.float32, "W")
    vec = W.dim() == 1
    W2 = W.view(1, -1) if vec else W
    N, K = W2.shape
    bits = torch.empty((N, K // 32), dtype=torch.int32, device=W.device)
    _call("tkq_pack_bin", _ptr(W2), N, K, _ptr(bits), _stream(stream, bits))
    return bits.view(-1) if vec else bits


def pack_int2_g128(W, stream=None):
    """W fp32 [N,K] -> (codes int32 [N,K/16], meta int32 [N,K/128] = half2 {s,z})."""
    _need(W, torch.float32, "W")
    N, K = W.shape
    codes = torch.empty((N, K // 16), dtype=torch.int32, device=W.device)
    meta = torch.empty((N, K // 128), dtype=torch.int32, device=W.device)
    _call("tkq_pack_int2_g128", _ptr(W), N, K, _ptr(codes), _ptr(meta), _stream(stream, codes, meta))
    return codes, meta


def pack_int3_g128(W, stream=None):
    """W fp32 [N,K] -> (codes int32 [3,N,K/32] (plane-major layout), meta int32 [N,K/128])."""
    _need(W, torch.float32, "W")
    N, K = W.shape
    codes = torch.empty((3, N, K // 32), dtype=torch.int32, device=W.device)
    meta = torch.empty((N, K // 128), dtype=torch.int32, device=W.device)
    _call("tkq_pack_int3_g128", _ptr(W), N, K, _ptr(codes), _ptr(meta), _stream(stream, codes, meta))
    return codes, meta


def hier_meta_bytes(N, K):
    """Size of an int4-hier-g32 metadata block (tkq_hier_meta_bytes)."""
    n = lib().tkq_hier_meta_bytes(N, K)
    if n < 0:
        raise TkqError(ESHAPE, "tkq_hier_meta_bytes")
    return n


def pack_int4_hier_g32(W, stream=None):
    """W fp32 [N,K] -> (codes int32 [N,K/8], meta uint8 [hier_meta_bytes(N,K)]):
    group bytes sc | mi << 4, zero padding, then half2 {d, dmin} per row."""
    _need(W, torch.float32, "W")
    N, K = W.shape
    codes = torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    meta = torch.empty(hier_meta_bytes(N, K), dtype=torch.uint8, device=W.device)
    _call("tkq_pack_int4_hier_g32", _ptr(W), N, K, _ptr(codes), _ptr(meta), _stream(stream, codes, meta))
    return codes, meta


PACKERS = {FMT_INT4_G128: pack_int4_g128, FMT_K5_G128: pack_k5,
           FMT_TERN_G128: pack_tern_g128, FMT_INT4_HIER_G32: pack_int4_hier_g32,
           FMT_INT2_G128: pack_int2_g128, FMT_INT3_G128: pack_int3_g128}


# ---- grouped GEMV ------------------------------------------------------------

class GemvBatch:
    """A prepared grouped GEMV: many y_i = dequant(W_i) . x_i in one launch.

    items: sequence of dicts with keys codes, meta (None for binary), x, y,
    N, K (tensors already on the device).  The descriptor table is built,
    planned by tkq_gemv_prepare and copied to the device once; run() launches
    tkq_gemv on the current (or given) stream."""

    def __init__(self, fmt, items, device=None, tokens=None):
        """tokens: None for the batch-1 GEMV (x [K], y [N]); M in 1..16 for
        the multi-token GEMV (x [M, K], y [M, N]; int4 g128 or int4-hier-g32)."""
        fmt = FORMATS.get(fmt, fmt)
        items = list(items)
        if not items:
            raise ValueError("empty GEMV batch")
        n = len(items)
        descs = (GemvDesc * n)()
        self._keep = []
        for d, it in zip(descs, items):
            d.fmt, d.N, d.K = fmt, int(it["N"]), int(it["K"])
            for key in ("codes", "meta", "x", "y"):
                t = it.get(key)
                if t is None:
                    setattr(d, key, None)
                    continue
                if not t.is_cuda or not t.is_contiguous():
                    raise ValueError("%s must be a contiguous device tensor" % key)
                setattr(d, key, t.data_ptr())
                self._keep.append(t)
        self.plan = GemvPlan()
        self.tokens = tokens
        if tokens is None:
            _call("tkq_gemv_prepare", descs, n, ctypes.byref(self.plan))
        else:
            _call("tkq_gemm_small_prepare", descs, n, int(tokens), ctypes.byref(self.plan))
        self.descs = descs
        raw = bytes(ctypes.string_at(ctypes.addressof(descs), ctypes.sizeof(descs)))
        dev = device if device is not None else self._keep[0].device
        self.dev_descs = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(dev)
        self.fmt, self.count, self.tiles = fmt, n, int(self.plan.tiles)

    def run(self, stream=None):
        if self.tokens is None:
            _call("tkq_gemv", ctypes.byref(self.plan), _ptr(self.dev_descs), _stream(stream, self.dev_descs))
        else:
            _call("tkq_gemm_small", ctypes.byref(self.plan), _ptr(self.dev_descs),
                  _stream(stream, self.dev_descs))

    def greedy_scratch(self):
        """Scratch for run_argmax: one int64 per tile of the launch."""
        return torch.empty(self.tiles, dtype=torch.int64, device=self.dev_descs.device)

    def run_argmax(self, target, token, scratch, stream=None):
        """run() plus the index of the largest output of item `target` into
        token (int32 device tensor, 1 element); scratch: greedy_scratch()."""
        _need(token, torch.int32, "token")
        _need(scratch, torch.int64, "scratch")
        _call("tkq_gemv_argmax", ctypes.byref(self.plan), _ptr(self.dev_descs), int(target),
              _ptr(token), _ptr(scratch), scratch.numel() * 8, _stream(stream, self.dev_descs))

    def run_argmax_static(self, target, token, stream=None):
        """run_argmax without caller scratch (tkq_gemv_argmax_static: the
        library's fixed per-device slot array; calls on one GPU must not
        overlap)."""
        _need(token, torch.int32, "token")
        _call("tkq_gemv_argmax_static", ctypes.byref(self.plan), _ptr(self.dev_descs), int(target),
              _ptr(token), _stream(stream, self.dev_descs))


    def run_argmax_rescore(self, target, head, k, token, scratch, cand=None, cand_logits=None, stream=None):
        """run() plus greedy selection with head rescore over item `target`
        (tkq_gemv_argmax_rescore): head is the fp16 copy [N, K] of the
        target's weights; token int32 [1]; scratch: greedy_scratch();
        cand int32 [k] and cand_logits float32 [k] optional."""
        d = self.descs[target]
        _need(head, torch.float16, "head", (d.N, d.K))
        _need(token, torch.int32, "token")
        _need(scratch, torch.int64, "scratch")
        if cand is not None:
            _need(cand, torch.int32, "cand", (k,))
        if cand_logits is not None:
            _need(cand_logits, torch.float32, "cand_logits", (k,))
        _call("tkq_gemv_argmax_rescore", ctypes.byref(self.plan), _ptr(self.dev_descs), int(target), d.N, d.K,
              _ptr(head), int(k), _ptr(token), _ptr(cand) if cand is not None else None,
              _ptr(cand_logits) if cand_logits is not None else None, _ptr(scratch), scratch.numel() * 8,
              _stream(stream, self.dev_descs))


def gemv(fmt, codes, meta, x, N, K, y=None, stream=None):
    """Single GEMV y = dequant(W) . x (binary: K - 2 popcount(W ^ x), int32)."""
    fmt = FORMATS.get(fmt, fmt)
    owned = None
    if y is None:
        dt = torch.int32 if fmt == FMT_BIN else torch.float16
        y = owned = torch.empty(N, dtype=dt, device=codes.device)
    _stream(stream, owned)
    GemvBatch(fmt, [dict(codes=codes, meta=meta, x=x, y=y, N=N, K=K)]).run(stream)
    return y


# ---- greedy selection with head rescore -------------------------------------

def head_rescore(logits, head, x, k, token=None, cand=None, cand_logits=None, stream=None):
    """tkq_head_rescore: the k largest stored logits (fp16 [n]) are computed
    again from the fp16 head copy ([n, K]) and x (fp16 [K]); returns the token
    (int32 device tensor, 1 element).  cand (int32 [k]) and cand_logits
    (float32 [k]) receive the candidate rows in greedy order and their
    recomputed logits when given."""
    _need(logits, torch.float16, "logits")
    n = logits.numel()
    _need(head, torch.float16, "head")
    if head.dim() != 2 or head.shape[0] != n:
        raise ValueError("head must be [n, K] with n = logits.numel()")
    K = head.shape[1]
    _need(x, torch.float16, "x", (K,))
    owned = None
    if token is None:
        token = owned = torch.empty(1, dtype=torch.int32, device=logits.device)
    _need(token, torch.int32, "token")
    if cand is not None:
        _need(cand, torch.int32, "cand", (k,))
    if cand_logits is not None:
        _need(cand_logits, torch.float32, "cand_logits", (k,))
    _call("tkq_head_rescore", _ptr(logits), n, _ptr(head), _ptr(x), K, int(k), _ptr(token),
          _ptr(cand) if cand is not None else None,
          _ptr(cand_logits) if cand_logits is not None else None, _stream(stream, owned))
    return token


# ---- prefill GEMM --------------------------------------------------------------

def gemm_prefill(codes, meta, X, N, Y=None, workspace=None, stream=None):
    """Y fp16 [M,N] = X fp16 [M,K] . dequant(W_int4_g128)^T.

    workspace: optional float32 device tensor; with >= 2*M*N elements the
    library may split K and use it for fp32 partial products."""
    _need(X, torch.float16, "X")
    M, K = X.shape
    _need(codes, torch.int32, "codes", (N, K // 8))
    _need(meta, torch.int32, "meta", (N, K // 128))
    owned = None
    if Y is None:
        Y = owned = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _need(Y, torch.float16, "Y", (M, N))
    ws, wsb = None, 0
    if workspace is not None:
        _need(workspace, torch.float32, "workspace")
        ws, wsb = _ptr(workspace), workspace.numel() * 4
    _call("tkq_gemm_prefill", FMT_INT4_G128, M, N, K, _ptr(codes), _ptr(meta), _ptr(X), _ptr(Y),
          ws, wsb, _stream(stream, owned))
    return Y


def read_probe(buf, out=None, stream=None):
    """Stream `buf` once with 16-byte non-temporal loads (bandwidth reference)."""
    owned = None
    if out is None:
        out = owned = torch.zeros(4, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _call("tkq_read_probe", _ptr(buf), nbytes, _ptr(out), _stream(stream, owned))
    return out


# ---- low-bit KV cache decode attention ------------------------------------------

def _seqlens(seqlens, B, device):
    if seqlens is None:
        return None
    _need(seqlens, torch.int32, "seqlens", (B,))
    if seqlens.device != device:
        raise ValueError("seqlens must be on the cache's device")
    return seqlens


def kv_pack(K, V, seqlens=None, stream=None):
    """K, V fp16 [B, T, Hk, 128] -> paged 4-bit cache (uint8 tensor of
    tkq_kv_cache_bytes bytes, viewed as [B, Hk, T/128, 17408]).  seqlens:
    optional int32 [B] device tensor of valid tokens per sequence
    (tkq_kv_pack_varlen: tokens past a length are packed as zeros)."""
    _need(K, torch.float16, "K")
    _need(V, torch.float16, "V", K.shape)
    B, T, Hk, D = K.shape
    n = lib().tkq_kv_cache_bytes(B, Hk, T)
    if n < 0 or D != 128:
        raise TkqError(ESHAPE, "tkq_kv_cache_bytes")
    cache = torch.empty(n, dtype=torch.uint8, device=K.device)
    lens = _seqlens(seqlens, B, K.device)
    if lens is None:
        _call("tkq_kv_pack", _ptr(K), _ptr(V), B, T, Hk, D, _ptr(cache), _stream(stream, cache))
    else:
        _call("tkq_kv_pack_varlen", _ptr(K), _ptr(V), _ptr(lens), B, T, Hk, D, _ptr(cache), _stream(stream, cache))
    return cache.view(B, Hk, T // 128, 17408)


def kv_workspace(B, H, Hk, T, device):
    """A zero-filled decode workspace (tkq_kv_decode_workspace_bytes)."""
    nws = lib().tkq_kv_decode_workspace_bytes(B, H, Hk, T)
    if nws < 0:
        raise TkqError(ESHAPE, "tkq_kv_decode_workspace_bytes")
    return torch.zeros((nws + 3) // 4, dtype=torch.float32, device=device)


def kv_decode(q, cache, T, sm_scale, seqlens=None, out=None, workspace=None, stream=None):
    """q fp16 [B, H, 128] -> out fp16 [B, H, 128] over a cache from kv_pack
    (seqlens: optional int32 [B] device tensor, tkq_kv_decode_varlen).
    workspace: from kv_workspace (zero-filled before its first use)."""
    _need(q, torch.float16, "q")
    B, H, D = q.shape
    Hk = cache.shape[1]
    owned = []
    if out is None:
        out = torch.empty_like(q)
        owned.append(out)
    _need(out, torch.float16, "out", q.shape)
    if workspace is None:
        workspace = kv_workspace(B, H, Hk, T, q.device)
        owned.append(workspace)
    _need(workspace, torch.float32, "workspace")
    lens = _seqlens(seqlens, B, q.device)
    if lens is None:
        _call("tkq_kv_decode", _ptr(q), _ptr(cache), B, H, Hk, T, D, float(sm_scale), _ptr(out), _ptr(workspace),
              workspace.numel() * 4, _stream(stream, *owned))
    else:
        _call("tkq_kv_decode_varlen", _ptr(q), _ptr(cache), _ptr(lens), B, H, Hk, T, D, float(sm_scale), _ptr(out),
              _ptr(workspace), workspace.numel() * 4, _stream(stream, *owned))
    return out


class KvDecoder:
    """A prepared tkq_kv_decode call (arguments marshalled once; run() is one
    C call), for decode loops where the per-call Python cost matters."""

    def __init__(self, q, cache, T, sm_scale, out=None, workspace=None, seqlens=None, stream=None):
        _need(q, torch.float16, "q")
        B, H, D = q.shape
        Hk = cache.shape[1]
        owned = []
        self.out = out if out is not None else torch.empty_like(q)
        if out is None:
            owned.append(self.out)
        _need(self.out, torch.float16, "out", q.shape)
        self.workspace = workspace if workspace is not None else kv_workspace(B, H, Hk, T, q.device)
        if workspace is None:
            owned.append(self.workspace)
        _need(self.workspace, torch.float32, "workspace")
        lens = _seqlens(seqlens, B, q.device)
        self._keep = (q, cache, lens)
        args = (_ptr(q), _ptr(cache)) + ((_ptr(lens),) if lens is not None else ()) + (
            B, H, Hk, T, D, ctypes.c_float(sm_scale), _ptr(self.out), _ptr(self.workspace),
            self.workspace.numel() * 4)
        self._args = args
        self._stream = _stream(stream, *owned)
        self._name = "tkq_kv_decode" if lens is None else "tkq_kv_decode_varlen"
        self._fn = getattr(lib(), self._name)

    def run(self):
        st = self._fn(*self._args, self._stream)
        if st != OK:
            raise TkqError(st, self._name)
        return self.out

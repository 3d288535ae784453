"""Benchmark of the low-bit GEMV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one decode-equivalent weight sweep: every linear layer a Qwen2.5
model reads per token, y_i = dequant(W_i) . x_i for all i, as ONE grouped
kernel launch.  Default workload: the Qwen2.5-0.5B sweep (169 GEMVs) in the
int4-g128 coding.  The timed region is exactly K steps between two stream
synchronisations; packed weights are resident in HBM and rotated over enough
distinct copies (>= 1 GiB in total) that no step is served from the 256 MB
Infinity Cache.  One JSON line goes to stdout.

value = algorithmic bytes per step (packed codes + fp16 metadata + x + y, each
once) / measured time per step, in TB/s.  The roofline object reports the
same kernel against the 8 TB/s HBM peak; cpu_baseline times the numpy oracle
on a bounded sample of the same workload on the host cores.

Other workloads (for measurement; each prints its own line): the 0.5B sweep
in the other codings (0.5b-k5, 0.5b-tern, 0.5b-hier, 0.5b-int2, 0.5b-int3),
with the greedy token (0.5b-int4-greedy) or the head rescore
(0.5b-int4-rescore, --rescore-k candidates), for M tokens at once
(0.5b-int4-mM, M = 2, 4, 8, 16; 7b-int4-m16; int4-hier-g32: 0.5b-hier-m16,
7b-hier-m16), the binary shapes (bin), the 7B
sweep (7b-int4, 7b-hier), the 7B MLP prefill (7b-prefill), KV-cache decode
(kv-4k, kv-32k, kv-32k-gqa, kv-128k-gqa), one 896 x 896 GEMV (single-896) and
the read probe (probe).
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "int4-g128 GEMV achieved HBM TB/s (% of peak) + decode-equiv tok/s, batch 1"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix cores
ROTATE_BYTES = 1 << 30

# HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE passes (each
# scaled by what the counter reads for a 256 MiB device copy); see the
# summaries under profiles/.  Valid only for the kernel sources they were
# measured on: a workload's figure is reported while the sources of its
# kernel family hash to the value stored with it, else null.
_COMMON = ["gemm_tkq_gemv_amd/csrc/tkq_api.hip", "gemm_tkq_gemv_amd/csrc/device_common.h",
           "gemm_tkq_gemv_amd/csrc/kernels.h"]
TRAFFIC_SOURCES = {"gemv": ["gemm_tkq_gemv_amd/csrc/gemv.hip"] + _COMMON,
                   "small_m": ["gemm_tkq_gemv_amd/csrc/small_m.hip"] + _COMMON,
                   "prefill": ["gemm_tkq_gemv_amd/csrc/prefill.hip"] + _COMMON,
                   "kv": ["gemm_tkq_gemv_amd/csrc/kv.hip"] + _COMMON}
# workload -> (kernel family, bytes per launch, sha256[:16] of that family's sources)
TRAFFIC_BYTES = {"0.5b-int4": ("gemv", 266616382, "b6f6bd5552d3944b"),
                 "0.5b-k5": ("gemv", 506971706, "b6f6bd5552d3944b"),
                 "0.5b-tern": ("gemv", 135444579, "b6f6bd5552d3944b"),
                 "bin": ("gemv", 115068394, "b6f6bd5552d3944b"),
                 "7b-int4": ("gemv", 3781892473, "b6f6bd5552d3944b"),
                 "7b-prefill": ("prefill", 238651956, "c2541f1b6ffb18bc"),
                 "0.5b-hier": ("gemv", 268438052, "b6f6bd5552d3944b"),
                 "0.5b-int2": ("gemv", 143153278, "b6f6bd5552d3944b"),
                 "0.5b-int3": ("gemv", 206228152, "b6f6bd5552d3944b"),
                 "0.5b-int4-greedy": ("gemv", 266693011, "b6f6bd5552d3944b"),
                 "0.5b-int4-m16": ("small_m", 383039047, "84bc997abcf0d8f2"),
                 "0.5b-hier-m16": ("small_m", 387133073, "84bc997abcf0d8f2"),
                 "kv-32k": ("kv", 143489614, "96a6fe5bf66eaca8"),
                 "kv-4k": ("kv", 18430846, "96a6fe5bf66eaca8"),
                 "kv-32k-gqa": ("kv", 37219117, "96a6fe5bf66eaca8"),
                 "kv-128k-gqa": ("kv", 145439373, "96a6fe5bf66eaca8")}


def traffic_family(workload):
    if workload.startswith("kv-"):
        return "kv"
    if workload == "7b-prefill":
        return "prefill"
    if "-m" in workload and workload.split("-m")[-1].isdigit():
        return "small_m"
    return "gemv"


def source_hash(family):
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[family]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    e = TRAFFIC_BYTES.get(workload)
    if e is None or source_hash(e[0]) != e[2]:
        return None
    return e[1]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- workloads --

def _pack(tkq, fmt, Wd):
    if fmt == "int4":
        return tkq.pack_int4_g128(Wd)
    if fmt == "k5":
        return tkq.pack_k5(Wd)
    if fmt == "tern":
        return tkq.pack_tern_g128(Wd)
    if fmt == "hier":
        return tkq.pack_int4_hier_g32(Wd)
    if fmt == "int2":
        return tkq.pack_int2_g128(Wd)
    if fmt == "int3":
        return tkq.pack_int3_g128(Wd)
    return tkq.pack_bin(Wd), None


def build_sweep(torch, tkq, inputs, model, fmt):
    """Pack every matrix of the model's sweep; returns (items, shapes)."""
    shapes = inputs.sweep_shapes(model)
    items = []
    t0 = time.time()
    for i, (_, N, K) in enumerate(shapes):
        if model == "qwen2.5-7b":
            Wd = inputs.device_normal_matrix(torch, 5000 + i, N, K)
            x = inputs.sweep_x(model, i, K)
        else:
            W, x = inputs.sweep_matrix(model, i, N, K)
            Wd = torch.from_numpy(W).cuda()
        codes, meta = _pack(tkq, fmt, Wd)
        del Wd
        y = torch.empty(N, dtype=torch.float16, device="cuda")
        items.append(dict(codes=codes, meta=meta, x=torch.from_numpy(x).cuda(), y=y, N=N, K=K))
    torch.cuda.synchronize()
    log("packed %s %s sweep: %d matrices in %.1f s" % (model, fmt, len(items), time.time() - t0))
    return items, shapes


def launch_groups(shapes, launch):
    """Index groups of the sweep, one GEMV launch per group: "grouped" = the
    whole sweep in one launch; "staged" = per layer q,k,v | o | gate,up |
    down, then the output projection (4 * layers + 1 launches); "per-matrix"
    = one launch per matrix."""
    n = len(shapes)
    if launch == "grouped":
        return [list(range(n))]
    if launch == "per-matrix":
        return [[i] for i in range(n)]
    groups = []
    for i0 in range(0, n - 1, 7):    # q k v o gate up down of one layer
        groups += [[i0, i0 + 1, i0 + 2], [i0 + 3], [i0 + 4, i0 + 5], [i0 + 6]]
    return groups + [[n - 1]]


def rotated_batches(torch, tkq, fmt, items, footprint, copies=None, launch="grouped", shapes=None):
    """Distinct copies of the packed weights (>= 1 GiB total unless `copies`
    is given; 1 = cache-resident), each a list of prepared launches."""
    if copies is None:
        copies = max(1, math.ceil(ROTATE_BYTES / footprint))
    groups = launch_groups(shapes, launch) if shapes is not None else [list(range(len(items)))]
    out = []
    for c in range(copies):
        its = items if c == 0 else [dict(it, codes=it["codes"].clone(),
                                         meta=None if it["meta"] is None else it["meta"].clone()) for it in items]
        out.append([tkq.GemvBatch(fmt, [its[i] for i in g]) for g in groups])
    torch.cuda.synchronize()
    return out


SWEEP_STATS = {}


def time_steps(torch, run_step, steps, warmup, graph="none", period=1, group=10):
    """Warm up, then time exactly `steps` steps between synchronisations with
    HIP events recorded on the stream the kernels are launched on.

    graph="step": each of the `period` distinct steps (rotation copies) is
    captured once as a HIP graph and step s replays graph s % period;
    graph="all": the `steps` timed steps are captured as one graph that is
    replayed once inside the timed region (warm-up steps run eagerly).
    Without "all", an event every `group` steps (and the end event for the
    last group) also gives the per-step median, p10 and p90 over the groups
    (SWEEP_STATS)."""
    for s in range(warmup):
        run_step(s)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    marks = []
    if graph == "none":
        start.record(stream)
        for s in range(steps):
            run_step(s)
            if (s + 1) % group == 0 and s + 1 < steps:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                marks.append(e)
        end.record(stream)
    elif graph == "step":
        graphs = []
        for p in range(period):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_step(p)
            graphs.append(g)
        torch.cuda.synchronize()
        start.record(stream)
        for s in range(steps):
            graphs[s % period].replay()
            if (s + 1) % group == 0 and s + 1 < steps:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                marks.append(e)
        end.record(stream)
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(steps):
                run_step(s)
        torch.cuda.synchronize()
        start.record(stream)
        g.replay()
        end.record(stream)
    torch.cuda.synchronize()
    SWEEP_STATS.clear()
    if marks:
        # every group enters the statistics, the last one (up to `group`
        # steps, closed by the end event) included
        pts = [start] + marks + [end]
        sizes = [group] * len(marks) + [steps - group * len(marks)]
        per = sorted(a.elapsed_time(b) / n for (a, b), n in zip(zip(pts, pts[1:]), sizes))
        q = lambda f: per[min(len(per) - 1, int(f * len(per)))]  # noqa: E731
        SWEEP_STATS.update(median_us=round(q(0.5) * 1e3, 3), p10_us=round(q(0.1) * 1e3, 3),
                           p90_us=round(q(0.9) * 1e3, 3), groups=len(per), steps_per_group=group)
    return start.elapsed_time(end) / steps  # ms per step


# ------------------------------------------------------------- cpu baseline --

def cpu_baseline_gemv(inputs, model, fmt, budget_s=10.0, M=None):
    """Oracle (numpy, fp64) timed on the host: dequantize the stored codes and
    run the fp64 matvec (M tokens: the fp64 product X . W^T).  The sample is
    the sweep's matrices in order (the 7B head truncated to its first 32768
    rows, its other matrices as they come) until ~20 s of preparation; then
    passes over the prepared sample are timed until `budget_s` seconds of
    oracle work.  Quantization and packing are not timed.  Rate =
    algorithmic bytes (weights once, x and y per token) / time."""
    import numpy as np

    from oracle import accounting, pack, quant, ref

    shapes = inputs.sweep_shapes(model)
    prepared, names, t_prep = [], [], time.perf_counter()
    for i, (name, N, K) in enumerate(shapes):
        if time.perf_counter() - t_prep > 20.0:
            break
        if model == "qwen2.5-7b":
            if N > 32768:
                N = 32768
            W = inputs.normal_matrix((5000, i), N, K)
            x = inputs.sweep_x(model, i, K)
        else:
            W, x = inputs.sweep_matrix(model, i, N, K)
        if M is not None:
            x = np.stack([inputs.normal_vector((6, i, m), K) for m in range(M)])
        if fmt == "int4":
            q, s, z = quant.quantize_int4_g128(W)
            prepared.append((fmt, (pack.pack_int4(q), pack.pack_int4_meta(s, z)), x, N, K))
        elif fmt == "k5":
            prepared.append((fmt, quant.quantize_k5(W), x, N, K))
        elif fmt == "int2":
            q, s, z = quant.quantize_int2_g128(W)
            prepared.append((fmt, (pack.pack_int2(q), pack.pack_int4_meta(s, z)), x, N, K))
        elif fmt == "int3":
            q, s, z = quant.quantize_int3_g128(W)
            prepared.append((fmt, (pack.pack_int3(q), pack.pack_int4_meta(s, z)), x, N, K))
        elif fmt == "hier":
            q, sc, mi, d16, dmin16 = quant.quantize_int4_hier_g32(W)
            prepared.append((fmt, (pack.pack_int4(q), pack.pack_hier_meta(sc, mi, d16, dmin16)), x, N, K))
        else:
            c, s = quant.quantize_tern_g128(W)
            prepared.append((fmt, (pack.pack_tern(c), s), x, N, K))
        names.append(name if N == shapes[i][1] else "%s[:%d]" % (name, N))
        del W

    def one(item):
        f, (c, m), x, N, K = item
        if f == "int4":
            w = ref.dequant_int4(c, m, K)
        elif f == "k5":
            w = ref.dequant_k5(c, m)
        elif f == "hier":
            w = ref.dequant_int4_hier(c, m, N, K)
        elif f == "int2":
            w = ref.dequant_int2(c, m, K)
        elif f == "int3":
            w = ref.dequant_int3(c, m, K)
        else:
            w = ref.dequant_tern(c, m, K)
        y = ref.gemv(w, x) if x.ndim == 1 else ref.gemm(x, w)
        assert np.all(np.isfinite(y))
        weights = accounting.gemv_bytes(f, N, K) - 2 * K - 2 * N
        return weights + (1 if x.ndim == 1 else x.shape[0]) * (2 * K + 2 * N)

    done_bytes, spent, passes = _cpu_loop(lambda: sum(one(it) for it in prepared), budget_s)
    return done_bytes / spent, spent, names, passes


def gemv_cpu_entry(inputs, model, fmt, budget_s, M=None):
    rate, spent, done, passes = cpu_baseline_gemv(inputs, model, fmt, budget_s, M)
    return _cpu_entry(round(rate / 1e12, 8), "TB/s",
                      "numpy oracle dequantize + fp64 %s, %d passes over the first %d matrices of the sweep "
                      "(%s), %.1f s of CPU work; quantization not timed"
                      % ("matvec" if M is None else "product with %d tokens" % M, passes, len(done),
                         ", ".join(done[:3] + (["..."] if len(done) > 3 else []) + done[-1:]), spent))


def _cpu_loop(work, budget_s):
    """Call work() (which returns the units it did) until budget_s seconds
    have passed, at least once: (units, seconds, passes)."""
    done, passes, t0 = 0, 0, time.perf_counter()
    while True:
        done += work()
        passes += 1
        spent = time.perf_counter() - t0
        if spent >= budget_s:
            return done, spent, passes


def _cpu_entry(value, unit, sample):
    return {"value": value, "unit": unit, "cores": blas_threads(),
            "host_cores_available": len(os.sched_getaffinity(0)), "kind": "oracle", "sample": sample}


def cpu_baseline_rescore(inputs, model, k, budget_s):
    """Oracle output projection with head rescore, per token: dequantize the
    int4 head and multiply in fp64, then pick the k candidates from the
    stored (fp16-rounded) logits and recompute them from the fp16 copy
    (oracle.rescore); quantization not timed.  Rate = algorithmic bytes of
    the head GEMV and the rescore / time."""
    from oracle import pack, quant, ref, rescore
    shapes = inputs.sweep_shapes(model)
    i = len(shapes) - 1
    _, N, K = shapes[i]
    W, x = inputs.sweep_matrix(model, i, N, K)
    q, s_, z = quant.quantize_int4_g128(W)
    c, m = pack.pack_int4(q), pack.pack_int4_meta(s_, z)
    head16 = W.astype(np.float16)
    del W, q
    unit = _fmt_bytes("int4")(N, K) + rescore_bytes(N, K, k)

    def work():
        y = ref.gemv(ref.dequant_int4(c, m, K), x).astype(np.float16)
        rescore.head_rescore(y, head16, x, k)
        return unit
    done, spent, passes = _cpu_loop(work, budget_s)
    return _cpu_entry(round(done / spent / 1e12, 8), "TB/s",
                      "numpy oracle: int4 output projection (%d x %d) dequantize + fp64 matvec, then head "
                      "rescore of the %d largest stored logits, %d tokens, %.1f s of CPU work; quantization "
                      "not timed" % (N, K, k, passes, spent))


def cpu_baseline_binary(inputs, budget_s):
    """Oracle XOR-popcount GEMV (numpy bitwise_count on uint32 words) over the
    six binary shapes; packing not timed.  Rate = algorithmic bytes / time."""
    from oracle import pack, quant, ref
    prepared = []
    for N, K in inputs.BINARY_SHAPES:
        W, x = inputs.binary_case(N, K)
        prepared.append((pack.pack_bits(quant.sign_bits(W)), pack.pack_bits(quant.sign_bits(x[None, :]))[0], N, K))
    fb = _fmt_bytes("bin")

    def work():
        n = 0
        for wb, xb, N, K in prepared:
            ref.bin_gemv(wb, xb, K)
            n += fb(N, K)
        return n
    done, spent, passes = _cpu_loop(work, budget_s)
    return _cpu_entry(round(done / spent / 1e12, 8), "TB/s",
                      "numpy oracle XOR-popcount over all six binary shapes, %d passes, %.1f s of CPU work; "
                      "packing not timed" % (passes, spent))


def cpu_baseline_prefill(inputs, budget_s):
    """Oracle prefill: dequantize the int4 gate, up and down weights to fp64
    and multiply by X in fp64 (the whole step, M = 512); quantization not
    timed.  Rate = step FLOP / time."""
    from oracle import pack, quant, ref
    M = inputs.PREFILL_M
    prepared = []
    for name, N, K in inputs.prefill_shapes():
        q, s_, z = quant.quantize_int4_g128(inputs.prefill_W(name))
        prepared.append((pack.pack_int4(q), pack.pack_int4_meta(s_, z), inputs.prefill_X(K).astype(np.float64), N, K))

    def work():
        f = 0
        for c, m, X, N, K in prepared:
            ref.gemm(X, ref.dequant_int4(c, m, K))
            f += 2 * M * N * K
        return f
    done, spent, passes = _cpu_loop(work, budget_s)
    return _cpu_entry(round(done / spent / 1e12, 6), "TFLOP/s",
                      "numpy oracle fp64 dequantize + fp64 matmul of the whole step (gate, up, down at M = 512), "
                      "%d passes, %.1f s of CPU work; quantization not timed" % (passes, spent))


def cpu_baseline_kv(inputs, B, H, Hk, T, budget_s):
    """Oracle decode attention (dequantize the cache pages to fp64, fp64
    softmax attention) on one KV head of the workload and its query heads;
    packing not timed.  Rate = bytes of that head's cache (+ q, out) / time."""
    from oracle import kv
    K, V, q = inputs.kv_random_case(B, H, Hk, T)
    G = H // Hk
    cache = kv.pack_cache(K[:1, :, :1], V[:1, :, :1])
    qs = q[:1, :G].astype(np.float64)
    nbytes = cache.nbytes + 2 * 2 * G * 128

    def work():
        Kd, Vd = kv.dequant_cache(cache)
        kv.attention_decode(qs, Kd, Vd, 1 / math.sqrt(128))
        return nbytes
    done, spent, passes = _cpu_loop(work, budget_s)
    return _cpu_entry(round(done / spent / 1e12, 8), "TB/s",
                      "numpy oracle page dequantization + fp64 attention for KV head 0 of sequence 0 (%d query "
                      "heads, %d tokens), %d passes, %.1f s of CPU work; packing not timed" % (G, T, passes, spent))


def cpu_baseline_single(inputs, budget_s):
    """Oracle 896 x 896 int4 GEMV: dequantize + fp64 matvec, per call."""
    from oracle import pack, quant, ref
    W, x = inputs.single_gemv_896()
    q, s_, z = quant.quantize_int4_g128(W)
    c, m = pack.pack_int4(q), pack.pack_int4_meta(s_, z)
    done, spent, passes = _cpu_loop(lambda: (ref.gemv(ref.dequant_int4(c, m, 896), x), 1)[1], budget_s)
    return _cpu_entry(round(spent / done * 1e6, 3), "us",
                      "numpy oracle dequantize + fp64 matvec of the 896x896 GEMV, %d calls, %.1f s of CPU work"
                      % (done, spent))


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return 1


# ------------------------------------------------------------------- runners --

def rescore_bytes(n, K, k):
    """Algorithmic bytes of one head rescore: the stored fp16 logits once, the
    k candidate rows of the fp16 head copy, x, and the token."""
    return 2 * n + 2 * k * K + 2 * K + 4


def run_sweep(args, torch, tkq, inputs, model, fmt, greedy=False, rescore_k=0):
    """greedy: the launch also selects the largest output of the last GEMV
    (the output projection) into a device token (tkq_gemv_argmax).
    rescore_k > 0: after the sweep, tkq_head_rescore recomputes the k largest
    stored logits of the output projection from an fp16 copy of it."""
    items, shapes = build_sweep(torch, tkq, inputs, model, fmt)
    fmt_bytes = _fmt_bytes(fmt)
    step_bytes = sum(fmt_bytes(n, k) for _, n, k in shapes)
    last = len(items) - 1
    if rescore_k:
        _, Nh, Kh = shapes[last]
        Wh, _ = inputs.sweep_matrix(model, last, Nh, Kh)
        head16 = torch.from_numpy(Wh).cuda().half().contiguous()
        del Wh
        step_bytes += rescore_bytes(Nh, Kh, rescore_k)
    footprint = sum(it["codes"].numel() * it["codes"].element_size()
                    + (0 if it["meta"] is None else it["meta"].numel() * it["meta"].element_size())
                    for it in items)
    launch = "grouped" if (greedy or rescore_k) else args.launch
    batches = rotated_batches(torch, tkq, fmt, items, footprint, args.copies, launch, shapes)
    rescore_us = None
    if greedy:
        token = torch.zeros(1, dtype=torch.int32, device="cuda")
        scratch = batches[0][0].greedy_scratch()
        step = lambda s: batches[s % len(batches)][0].run_argmax(last, token, scratch)  # noqa: E731
    elif rescore_k:
        token = torch.zeros(1, dtype=torch.int32, device="cuda")
        yh, xh = items[last]["y"], items[last]["x"]   # shared by every weight copy
        if args.rescore_path == "fused":   # the GEMV stores per-tile keys, the rescore starts from them
            scratch = batches[0][0].greedy_scratch()
            step = lambda s: batches[s % len(batches)][0].run_argmax_rescore(  # noqa: E731
                last, head16, rescore_k, token, scratch)
        else:
            def step(s):
                batches[s % len(batches)][0].run()
                tkq.head_rescore(yh, head16, xh, rescore_k, token=token)
    else:
        def step(s):
            for b in batches[s % len(batches)]:
                b.run()
    ms = time_steps(torch, step, args.steps, args.warmup, args.graph, len(batches))
    sweep_stats = dict(SWEEP_STATS)
    if rescore_k:   # the standalone rescore kernel alone, on the last sweep's logits
        rescore_us = round(1000.0 * time_steps(
            torch, lambda s: tkq.head_rescore(yh, head16, xh, rescore_k, token=token), 200, 20), 3)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    ceiling_tok_s = HBM_PEAK_GBS * 1e9 / step_bytes
    out = {
        "metric": METRIC if fmt == "int4" else "%s GEMV achieved HBM TB/s + decode-equiv tok/s, batch 1" % fmt,
        "value": round(gbs / 1000.0, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic: seeded N(0,0.02) weights at the model's shapes, N(0,1) fp16 x",
        "config": {"workload": "%s decode weight sweep, %s, %d GEMVs %s, batch 1%s"
                               % (model, _fmt_name(fmt), len(shapes),
                                  {"grouped": "in one launch",
                                   "staged": "in %d launches (per layer q,k,v | o | gate,up | down, then the "
                                             "output projection)" % len(batches[0]),
                                   "per-matrix": "in one launch each"}[launch],
                                  ", greedy token selected on the GPU in the same launch" if greedy else
                                  (", then greedy selection with head rescore (the %d largest stored logits of "
                                   "the output projection recomputed from its fp16 copy; %s)"
                                   % (rescore_k, "candidates from the GEMV's per-tile keys"
                                      if args.rescore_path == "fused" else "candidates from the stored logits")
                                   if rescore_k else "")),
                   "bytes_per_step": step_bytes, "copies_rotated": len(batches),
                   "cache_resident": len(batches) == 1 and args.copies == 1,
                   "weights": _fmt_name(fmt), "x": "fp16", "accumulate": "fp32", "y": "fp16",
                   "launch": launch + (", hip graph replay" if args.graph != "none" else ", stream launch")},
        "sweep_us": sweep_stats,
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tok_s": round(1000.0 / ms, 1), "ceiling_tok_s": round(ceiling_tok_s, 1),
        "frac_of_ceiling": round((1000.0 / ms) / ceiling_tok_s, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": args.traffic if args.traffic is not None else
                     (measured_traffic(args.workload) if launch == "grouped" and args.copies is None else None)},
        "kernel": (gemv_kernel_name(fmt, max(b.plan.variant for b in batches[0]),
                                    greedy or (rescore_k and args.rescore_path == "fused")).split(" + ")[0]
                   + (" + gemv_rescore_kernel" if rescore_k and args.rescore_path == "fused" else
                      " + head_rescore_kernel" if rescore_k else
                      " + greedy_finish_kernel" if greedy else "")),
    }
    if rescore_k:
        out["rescore"] = {"k": rescore_k, "path": args.rescore_path, "standalone_kernel_us": rescore_us,
                          "bytes": rescore_bytes(shapes[last][1], shapes[last][2], rescore_k),
                          "head_copy_bytes": 2 * shapes[last][1] * shapes[last][2]}
    del items, batches
    return out


SMALL_FMT_NAMES = {"int4": "int4-g128", "hier": "int4-hier-g32"}


def run_small(args, torch, tkq, inputs, model, M, fmt="int4"):
    """Multi-token GEMV: the model's whole sweep for M tokens at once
    (speculative verification of M draft tokens), int4 g128 or
    int4-hier-g32, one launch."""
    items, shapes = build_sweep(torch, tkq, inputs, model, fmt)
    for i, it in enumerate(items):
        K, N = it["K"], it["N"]
        X = np.stack([inputs.normal_vector((6, i, m), K) for m in range(M)])
        it["x"] = torch.from_numpy(X).cuda()
        it["y"] = torch.empty((M, N), dtype=torch.float16, device="cuda")
    # codes + metadata the kernel reads (the hier block's alignment padding is not read)
    weight_bytes = sum(n * k // 2 + n * k // 32 + (4 * n if fmt == "hier" else 0) for _, n, k in shapes)
    step_bytes = weight_bytes + sum(M * (2 * k + 2 * n) for _, n, k in shapes)
    flops = sum(2 * M * n * k for _, n, k in shapes)
    copies = max(1, math.ceil(ROTATE_BYTES / weight_bytes))
    batches = [tkq.GemvBatch(fmt, items, tokens=M)]
    for _ in range(copies - 1):
        clone = [dict(it, codes=it["codes"].clone(), meta=it["meta"].clone()) for it in items]
        batches.append(tkq.GemvBatch(fmt, clone, tokens=M))
    torch.cuda.synchronize()
    ms = time_steps(torch, lambda s: batches[s % len(batches)].run(), args.steps, args.warmup, args.graph,
                    len(batches))
    gbs = step_bytes / (ms * 1e-3) / 1e9
    name = SMALL_FMT_NAMES[fmt]
    return {"metric": "%s multi-token GEMV (M=%d) achieved HBM TB/s" % (name, M),
            "value": round(gbs / 1000.0, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f16",
            "data": "synthetic: seeded N(0,0.02) weights at the model's shapes, N(0,1) fp16 tokens",
            "config": {"workload": "%s weight sweep for %d tokens at once (%s, %d matrices, one launch)"
                                   % (model, M, name, len(shapes)),
                       "tokens": M, "bytes_per_step": step_bytes, "flops_per_step": flops,
                       "copies_rotated": len(batches)},
            "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "tok_s": round(M * 1000.0 / ms, 1),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload)},
            "kernel": "small_m_kernel"}


def run_kv(args, torch, tkq, B, H, Hk, T):
    """Single-query decode attention over a 4-bit paged KV cache (BitDecoding's
    shape: head dimension 128, group 128, K per channel, V per token)."""
    from gemm_tkq_gemv_amd import inputs
    Kh, Vh, qh = inputs.kv_random_case(B, H, Hk, T)
    caches = [tkq.kv_pack(torch.from_numpy(Kh).cuda(), torch.from_numpy(Vh).cuda())]
    del Kh, Vh
    cache_bytes = caches[0].numel()
    copies = max(1, math.ceil(ROTATE_BYTES / cache_bytes))
    for _ in range(copies - 1):
        caches.append(caches[0].clone())
    q = torch.from_numpy(qh).cuda()
    out = torch.empty_like(q)
    ws = tkq.kv_workspace(B, H, Hk, T, q.device)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(128)
    decs = [tkq.KvDecoder(q, c, T, scale, out, ws) for c in caches]
    ms = time_steps(torch, lambda s: decs[s % len(decs)].run(), args.steps, args.warmup, args.graph, len(decs))
    step_bytes = cache_bytes + 2 * 2 * B * H * 128
    gbs = step_bytes / (ms * 1e-3) / 1e9
    return {"metric": "4-bit KV-cache decode attention achieved HBM TB/s", "value": round(gbs / 1000.0, 4),
            "unit": "TB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
            "data": "synthetic N(0,1) fp16 K, V, q",
            "config": {"workload": "decode attention, batch %d, %d query / %d KV heads, head dim 128, %d cached "
                                   "tokens, 4-bit KV (K per channel, V per token, group 128)" % (B, H, Hk, T),
                       "bytes_per_step": step_bytes, "copies_rotated": len(caches)},
            "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload)},
            "kernel": "kv_decode_mfma_kernel" if H // Hk >= 3 else "kv_decode_kernel<%d>" % min(H // Hk, 8)}


def gemv_kernel_name(fmt, jmax, greedy):
    """The GEMV kernel instance a launch runs, as the profiler names it:
    int4 g128 has its own kernel, gemv_int4_kernel<greedy variant>; the other
    codings run gemv_kernel<coding, largest pass count, greedy variant>."""
    from gemm_tkq_gemv_amd import tkq
    flag = "true" if greedy else "false"
    name = ("gemv_int4_kernel<%s>" % flag if fmt == "int4"
            else "gemv_kernel<%d, %d, %s>" % (tkq.FORMATS[fmt], jmax, flag))
    return name + (" + greedy_finish_kernel" if greedy else "")


def _fmt_name(fmt):
    return {"int4": "int4-g128", "k5": "K5-g128", "tern": "ternary-g128 (2-bit)", "bin": "binary",
            "hier": "int4-hier-g32", "int2": "int2-g128", "int3": "int3-g128"}[fmt]


def _fmt_bytes(fmt):
    # codes + metadata + x + y per GEMV (the same accounting as the oracle's)
    return {
        "int4": lambda n, k: n * k // 2 + n * (k // 128) * 4 + 2 * k + 2 * n,
        "k5": lambda n, k: n * k + n * (k // 128) * 2 + 2 * k + 2 * n,
        "tern": lambda n, k: n * k // 4 + n * (k // 128) * 2 + 2 * k + 2 * n,
        "bin": lambda n, k: n * k // 8 + k // 8 + 4 * n,
        "hier": lambda n, k: n * k // 2 + n * (k // 32) + 4 * n + 2 * k + 2 * n,
        "int2": lambda n, k: n * k // 4 + n * (k // 128) * 4 + 2 * k + 2 * n,
        "int3": lambda n, k: 3 * n * k // 8 + n * (k // 128) * 4 + 2 * k + 2 * n,
    }[fmt]


def run_binary(args, torch, tkq, inputs):
    items = []
    for N, K in inputs.BINARY_SHAPES:
        W, x = inputs.binary_case(N, K)
        bits = tkq.pack_bin(torch.from_numpy(W).cuda())
        xb = tkq.pack_bin(torch.from_numpy(x).cuda())
        items.append(dict(codes=bits, meta=None, x=xb, y=torch.empty(N, dtype=torch.int32, device="cuda"),
                          N=N, K=K))
    step_bytes = sum(_fmt_bytes("bin")(n, k) for n, k in inputs.BINARY_SHAPES)
    footprint = sum(it["codes"].numel() * 4 for it in items)
    batches = [b[0] for b in rotated_batches(torch, tkq, "bin", items, footprint)]
    ms = time_steps(torch, lambda s: batches[s % len(batches)].run(), args.steps, args.warmup,
                    args.graph, len(batches))
    gbs = step_bytes / (ms * 1e-3) / 1e9
    return {"metric": "binary XOR-popcount GEMV achieved HBM TB/s", "value": round(gbs / 1000, 4),
            "unit": "TB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "u32", "data": "synthetic Bernoulli(0.5) signs",
            "config": {"workload": "binary sign GEMVs N in {896,4864,151936} x K in {896,4864}, one launch",
                       "bytes_per_step": step_bytes, "copies_rotated": len(batches)},
            "kernel": gemv_kernel_name("bin", batches[0].plan.variant, False),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("bin")}}


def run_single(args, torch, tkq, inputs):
    W, x = inputs.single_gemv_896()
    codes, meta = tkq.pack_int4_g128(torch.from_numpy(W).cuda())
    y = torch.empty(896, dtype=torch.float16, device="cuda")
    batch = tkq.GemvBatch("int4", [dict(codes=codes, meta=meta, x=torch.from_numpy(x).cuda(), y=y,
                                        N=896, K=896)])
    ms = time_steps(torch, lambda s: batch.run(), args.steps, args.warmup, args.graph, 1)
    b = _fmt_bytes("int4")(896, 896)
    return {"metric": "single int4-g128 896x896 GEMV latency", "value": round(ms * 1000, 3),
            "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": False, "scaling": "weak",
            "vs_baseline": None, "dtype": "f16", "data": "synthetic, seed 0",
            "config": {"workload": "single int4-g128 GEMV 896x896 (cache-resident, launch-bound)",
                       "bytes_per_step": b}}


def run_prefill(args, torch, tkq, inputs):
    """gate and up share X, so they run as one GEMM over the row-concatenated
    [gate; up] weights (N = 2 x 18944); down is a second GEMM.  A caller-owned
    fp32 workspace lets the library split K where that fills the GPU better."""
    Ws = {name: inputs.prefill_W(name) for name, _, _ in inputs.prefill_shapes()}
    M = inputs.PREFILL_M
    gemms = []
    for W in (np.concatenate([Ws["gate"], Ws["up"]]), Ws["down"]):
        N, K = W.shape
        codes, meta = tkq.pack_int4_g128(torch.from_numpy(W).cuda())
        X = torch.from_numpy(inputs.prefill_X(K)).cuda()
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        ws = torch.empty(8 * M * N, dtype=torch.float32, device="cuda")
        gemms.append((codes, meta, X, Y, N, ws))
    del Ws

    def step(_s):
        for codes, meta, X, Y, N, ws in gemms:
            tkq.gemm_prefill(codes, meta, X, N, Y, workspace=ws)

    ms = time_steps(torch, step, args.steps, args.warmup, args.graph, 1)
    flops = sum(2 * M * n * k for _, n, k in inputs.prefill_shapes())
    tf = flops / (ms * 1e-3) / 1e12
    return {"metric": "int4-g128 prefill GEMM (M=512) TFLOP/s", "value": round(tf, 2),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f16",
            "data": "synthetic N(0,0.02) weights, N(0,1) fp16 activations",
            "config": {"workload": "qwen2.5-7b MLP prefill, M=512, int4-g128 weights: gate+up as one "
                                   "GEMM (N=37888, K=3584) then down (N=3584, K=18944)",
                       "flops_per_step": flops},
            "tok_s": round(M * 1000.0 / ms, 1),
            "kernel": "prefill_kernel<8> (gate+up, then down) + tail_reduce_kernel + splitk_reduce_kernel",
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("7b-prefill")}}


def run_probe(args, torch, tkq, inputs):
    nbytes = 4 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    buf.fill_(1)
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    ms = time_steps(torch, lambda s: tkq.read_probe(buf, out), args.steps, args.warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"metric": "read-only stream probe HBM GB/s", "value": round(gbs, 1), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32",
            "data": "4 GiB buffer", "config": {"workload": "16-byte non-temporal read of 4 GiB"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="0.5b-int4",
                    choices=["0.5b-int4", "0.5b-int4-greedy", "0.5b-int4-rescore", "0.5b-k5", "0.5b-tern", "0.5b-hier",
                             "0.5b-int2", "0.5b-int3", "0.5b-int4-m2", "0.5b-int4-m4", "0.5b-int4-m8", "0.5b-int4-m16",
                             "7b-int4-m16", "0.5b-hier-m16", "7b-hier-m16", "kv-32k", "kv-32k-gqa", "kv-4k", "kv-128k-gqa", "bin", "single-896",
                             "7b-int4", "7b-hier", "7b-prefill", "probe"])
    ap.add_argument("--graph", default="none", choices=["none", "step", "all"],
                    help="launch steps as HIP graph replays (see time_steps)")
    ap.add_argument("--launch", default="grouped", choices=["grouped", "staged", "per-matrix"],
                    help="weight sweeps: one grouped launch (the measured path), per-layer stages, or one "
                         "launch per matrix (shows the launch cost; combine with --graph step)")
    ap.add_argument("--copies", type=int, default=None,
                    help="weight copies rotated (default: enough for >= 1 GiB; 1 = cache-resident)")
    ap.add_argument("--rescore-k", type=int, default=64,
                    help="candidates recomputed by the 0.5b-int4-rescore workload")
    ap.add_argument("--rescore-path", default="fused", choices=["fused", "standalone"],
                    help="0.5b-int4-rescore: tkq_gemv_argmax_rescore (fused) or tkq_gemv + tkq_head_rescore")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before anything else, copy a MIB-sized device buffer once (a kernel of "
                         "known traffic for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--traffic", type=float, default=None,
                    help="HBM bytes per launch from rocprofv3 FETCH_SIZE+WRITE_SIZE (scaled)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the batch-1 GEMV needs no collectives, and "
              "the library runs each launch on a single MI355X.  Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from gemm_tkq_gemv_amd import inputs, tkq
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    tkq.lib()
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration << 18, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    w = args.workload
    if w in ("0.5b-int4", "0.5b-int4-greedy", "0.5b-int4-rescore", "0.5b-k5", "0.5b-tern", "0.5b-hier",
             "0.5b-int2", "0.5b-int3", "7b-int4", "7b-hier"):
        model = "qwen2.5-7b" if w.startswith("7b") else "qwen2.5-0.5b"
        fmt = w.split("-")[1]
        rk = args.rescore_k if w.endswith("rescore") else 0
        out = run_sweep(args, torch, tkq, inputs, model, fmt, greedy=w.endswith("greedy"), rescore_k=rk)
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = (cpu_baseline_rescore(inputs, model, rk, args.cpu_budget) if rk else
                                   gemv_cpu_entry(inputs, model, fmt, args.cpu_budget))
    elif w.startswith("kv-"):
        T = {"4k": 4096, "32k": 32768, "128k": 131072}[w.split("-")[1]]
        Hk = 8 if w.endswith("gqa") else 32
        out = run_kv(args, torch, tkq, 1, 32, Hk, T)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_kv(inputs, 1, 32, Hk, T, args.cpu_budget)
    elif "-m" in w:
        model = "qwen2.5-7b" if w.startswith("7b") else "qwen2.5-0.5b"
        M = int(w.split("-m")[1])
        fmt = "hier" if "-hier-" in w else "int4"
        out = run_small(args, torch, tkq, inputs, model, M, fmt)
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = gemv_cpu_entry(inputs, model, fmt, args.cpu_budget, M)
    elif w == "bin":
        out = run_binary(args, torch, tkq, inputs)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_binary(inputs, args.cpu_budget)
    elif w == "single-896":
        out = run_single(args, torch, tkq, inputs)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_single(inputs, min(args.cpu_budget, 3.0))
    elif w == "7b-prefill":
        out = run_prefill(args, torch, tkq, inputs)
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_prefill(inputs, args.cpu_budget)
    else:
        out = run_probe(args, torch, tkq, inputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Seeded synthetic inputs and workload shapes.

This module holds no arithmetic of the method: it only draws random numbers
with numpy's PCG64 generator and lists matrix shapes.  Both the HIP path (via
the tests and the benchmark) and the CPU oracle consume the arrays it returns.

Recipes (all ``np.random.default_rng`` = PCG64, ``standard_normal`` drawn in
float32):

* single 896 x 896 GEMV: rng = default_rng(0); W = rng.standard_normal((896,
  896), float32) * float32(0.02); then x = rng.standard_normal(896,
  float32).astype(float16).
* Qwen2.5-shaped sweeps: matrix i (in the order L0.q, L0.k, L0.v, L0.o,
  L0.gate, L0.up, L0.down, L1.q, ..., lm_head) uses
  W_i = default_rng((cfg, i)).standard_normal((N, K), float32) * 0.02 and
  x_i = default_rng((cfg, 1000 + i)).standard_normal(K, float32) as float16,
  with cfg = 2 for the 0.5B model (x_i also for the 7B model, cfg = 5).
* binary sign GEMV (N, K): bits = default_rng((4, N, K)).integers(0, 2,
  (N, K)); W = 1 - 2*bits as float32; x bits from default_rng((4, N, K, 1)).
* Qwen2.5-7B sweep weights: drawn on the device, torch Philox seeded with
  5000 + i, N(0, 0.02); x_i as above with cfg = 5.
* prefill weights: default_rng((5, 4 | 5 | 6)) for gate / up / down,
  N(0, 0.02) float32 of the 7B MLP shapes.
* prefill activations: X = default_rng((5, 10000)) standard normal [512, 3584]
  float16 for gate/up and default_rng((5, 10001)) [512, 18944] for down.
* large-activation GEMV case (seed s, N, K): heavy-tailed weights
  0.02 * standard_t(3) with one outlier weight of magnitude 0.5..2 per
  group of 128 (position and sign drawn) and two activation channels per
  group set to +-A, A drawn from {1e3, 2e3, 4e3, 8e3, 3e4}, on which every
  row's weight is exactly 0 (so it quantizes to the zero point); the other
  activations are N(0, 1).  Decode activations have such outlier channels.
* KV cache, random: K, V, q standard normal fp16 ([B][T][Hk][128] and
  [B][H][128]), default_rng((9, B, H, Hk, T)) for the benchmark workloads.
* KV cache, page markers (B, H, Hk, T): K = 0, so every score ties and the
  attention is the plain mean over the cache; V[b, t, hk, c] = 15 on the
  marker channel c = (t // 128 + 37 hk + 11 b) % 128 of the token's page and
  1 elsewhere (exact on the 4-bit grid); q standard normal from
  default_rng((10, B, H, Hk, T)).  A page dropped, repeated, or read from
  another head or sequence moves its marker channel by about 14 / pages.
* KV cache, one peaked token (B, H, Hk, T, t): K and V standard normal fp16
  from default_rng((11, B, H, Hk, T)) with K scaled by 0.05, except that
  token t's K row is +4 in every channel of every KV head; q = +1, so token t
  dominates every head's softmax and the answer is its V row.
* KV cache, query outliers (B, H, Hk, T): K, V, q standard normal fp16 from
  default_rng((12, B, H, Hk, T)), except that channels 5, 37, 77 and 120 of
  K are 0 for every token (each such channel quantizes to its zero point)
  and carry query values of +-1e3, -3e3, +1e4 and -3e4 in every head.
  Queries have such outlier channels; their keys here dequantize to 0.

Shapes follow the Qwen2.5-0.5B (hidden 896, intermediate 4864, 24 layers,
2 KV heads x 64 = 128, vocab 151936, tied head) and Qwen2.5-7B (hidden 3584,
intermediate 18944, 28 layers, 4 KV heads x 128 = 512, vocab 152064)
configurations; weights are random stand-ins for trained checkpoints, since
the GEMV's time does not depend on the values.
"""

import numpy as np

QWEN05B = dict(hidden=896, inter=4864, layers=24, kv=128, vocab=151936)
QWEN7B = dict(hidden=3584, inter=18944, layers=28, kv=512, vocab=152064)
SWEEP_CFG = {"qwen2.5-0.5b": 2, "qwen2.5-7b": 5}
MODELS = {"qwen2.5-0.5b": QWEN05B, "qwen2.5-7b": QWEN7B}


def sweep_shapes(model="qwen2.5-0.5b"):
    """[(name, N, K)] of every linear layer read per decoded token, in order."""
    m = MODELS[model]
    h, f, kv = m["hidden"], m["inter"], m["kv"]
    out = []
    for layer in range(m["layers"]):
        for name, n, k in (("q", h, h), ("k", kv, h), ("v", kv, h), ("o", h, h),
                           ("gate", f, h), ("up", f, h), ("down", h, f)):
            out.append(("L%d.%s" % (layer, name), n, k))
    out.append(("lm_head", m["vocab"], h))
    return out


def single_gemv_896():
    """(W fp32 [896,896], x fp16 [896]) for the single-GEMV case, seed 0."""
    r = np.random.default_rng(0)
    W = r.standard_normal((896, 896), dtype=np.float32) * np.float32(0.02)
    x = r.standard_normal(896, dtype=np.float32).astype(np.float16)
    return W, x


def sweep_matrix(model, i, N, K):
    """(W fp32 [N,K], x fp16 [K]) of matrix i of a sweep."""
    cfg = SWEEP_CFG[model]
    W = np.random.default_rng((cfg, i)).standard_normal((N, K), dtype=np.float32)
    W *= np.float32(0.02)
    x = np.random.default_rng((cfg, 1000 + i)).standard_normal(K, dtype=np.float32)
    return W, x.astype(np.float16)


def sweep_weight_rows(model, i, N, K, rows):
    """Rows of W_i without materialising the whole matrix when it is large.

    PCG64 draws standard normals row-major, so row r needs the first r*K
    draws skipped; for simplicity this regenerates the matrix in chunks."""
    rows = np.asarray(rows, dtype=np.int64)
    cfg = SWEEP_CFG[model]
    r = np.random.default_rng((cfg, i))
    out = np.empty((rows.size, K), dtype=np.float32)
    order = np.argsort(rows)
    srt = rows[order]
    chunk = max(1, (64 << 20) // (4 * K))
    pos = 0
    j = 0
    while pos < N and j < srt.size:
        cnt = min(chunk, N - pos)
        blk = r.standard_normal((cnt, K), dtype=np.float32)
        while j < srt.size and srt[j] < pos + cnt:
            out[order[j]] = blk[srt[j] - pos]
            j += 1
        pos += cnt
    return out * np.float32(0.02)


def sweep_x(model, i, K):
    cfg = SWEEP_CFG[model]
    return np.random.default_rng((cfg, 1000 + i)).standard_normal(K, dtype=np.float32).astype(np.float16)


def binary_case(N, K):
    """(W {-1,+1} fp32 [N,K], x {-1,+1} fp32 [K]) for the sign GEMV."""
    bits = np.random.default_rng((4, N, K)).integers(0, 2, (N, K))
    xb = np.random.default_rng((4, N, K, 1)).integers(0, 2, K)
    return (1 - 2 * bits).astype(np.float32), (1 - 2 * xb).astype(np.float32)


BINARY_SHAPES = [(n, k) for n in (896, 4864, 151936) for k in (896, 4864)]


def prefill_shapes():
    """[(name, N, K)] of the M=512 prefill GEMMs (Qwen2.5-7B layer 0 MLP)."""
    m = QWEN7B
    return [("gate", m["inter"], m["hidden"]), ("up", m["inter"], m["hidden"]),
            ("down", m["hidden"], m["inter"])]


PREFILL_M = 512


def prefill_X(K, M=PREFILL_M):
    """fp16 activations [M, K]: seed (5, 10000) for K = 3584, (5, 10001) else."""
    seed = (5, 10000) if K == QWEN7B["hidden"] else (5, 10001)
    return np.random.default_rng(seed).standard_normal((M, K), dtype=np.float32).astype(np.float16)


def prefill_W(name):
    """7B-shaped MLP weights for the prefill GEMMs: numpy seeds (5, 4), (5, 5)
    and (5, 6) for gate, up and down (N(0, 0.02) float32)."""
    idx = {"gate": 4, "up": 5, "down": 6}[name]
    shapes = sweep_shapes("qwen2.5-7b")
    _, N, K = shapes[idx]
    W = np.random.default_rng((SWEEP_CFG["qwen2.5-7b"], idx)).standard_normal((N, K), dtype=np.float32)
    return W * np.float32(0.02)


def device_normal_matrix(torch, seed, N, K, std=0.02):
    """N(0, std) float32 [N, K] drawn on the GPU with torch's seeded Philox
    generator (used for the 7B-shaped sweep, whose 7.07 G weights take minutes
    to draw on the host).  `torch` is passed in so this module imports no GPU
    framework."""
    g = torch.Generator(device="cuda")
    g.manual_seed(int(seed))
    W = torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32)
    return W.mul_(std)


def normal_matrix(seed, N, K, std=0.02):
    """Small seeded test matrix: N(0, std) float32."""
    W = np.random.default_rng(seed).standard_normal((N, K), dtype=np.float32)
    return W * np.float32(std)


def normal_vector(seed, K):
    """Small seeded fp16 activation vector ~ N(0, 1)."""
    return np.random.default_rng(seed).standard_normal(K, dtype=np.float32).astype(np.float16)


def outlier_case(seed, N, K, group=128):
    """(W fp32 [N,K], x fp16 [K]): heavy-tailed weights with one outlier per
    group, and large activation channels on all-zero weight columns (the
    recipe above)."""
    r = np.random.default_rng(seed)
    W = (r.standard_t(3, (N, K)) * 0.02).astype(np.float32)
    x = r.standard_normal(K, dtype=np.float32)
    G = K // group
    out_pos = r.integers(0, group, (N, G))
    out_val = (r.uniform(0.5, 2.0, (N, G)) * r.choice([-1.0, 1.0], (N, G))).astype(np.float32)
    for g in range(G):
        W[np.arange(N), g * group + out_pos[:, g]] = out_val[:, g]
        chans = g * group + r.choice(group, 2, replace=False)
        W[:, chans] = 0.0
        x[chans] = r.choice([1e3, 2e3, 4e3, 8e3, 3e4], 2) * r.choice([-1.0, 1.0], 2)
    return W, x.astype(np.float16)


def kv_random_case(B, H, Hk, T, seed=9):
    """(K, V fp16 [B][T][Hk][128], q fp16 [B][H][128]), standard normal."""
    r = np.random.default_rng((seed, B, H, Hk, T))
    K = r.standard_normal((B, T, Hk, 128), dtype=np.float32).astype(np.float16)
    V = r.standard_normal((B, T, Hk, 128), dtype=np.float32).astype(np.float16)
    q = r.standard_normal((B, H, 128), dtype=np.float32).astype(np.float16)
    return K, V, q


def kv_marker_case(B, H, Hk, T):
    """(K, V, q) of the page-marker recipe above."""
    K = np.zeros((B, T, Hk, 128), np.float16)
    V = np.ones((B, T, Hk, 128), np.float16)
    page = np.arange(T) // 128
    for b in range(B):
        for hk in range(Hk):
            V[b, np.arange(T), hk, (page + 37 * hk + 11 * b) % 128] = 15
    q = np.random.default_rng((10, B, H, Hk, T)).standard_normal((B, H, 128), dtype=np.float32)
    return K, V, q.astype(np.float16)


def kv_peaked_case(B, H, Hk, T, t):
    """(K, V, q) of the one-peaked-token recipe above."""
    r = np.random.default_rng((11, B, H, Hk, T))
    K = (r.standard_normal((B, T, Hk, 128), dtype=np.float32) * np.float32(0.05)).astype(np.float16)
    V = r.standard_normal((B, T, Hk, 128), dtype=np.float32).astype(np.float16)
    K[:, t] = 4.0
    q = np.ones((B, H, 128), np.float16)
    return K, V, q


def kv_outlier_case(B, H, Hk, T):
    """(K, V, q) of the query-outlier recipe above."""
    r = np.random.default_rng((12, B, H, Hk, T))
    K = r.standard_normal((B, T, Hk, 128), dtype=np.float32).astype(np.float16)
    V = r.standard_normal((B, T, Hk, 128), dtype=np.float32).astype(np.float16)
    q = r.standard_normal((B, H, 128), dtype=np.float32)
    for c, a in zip((5, 37, 77, 120), (1e3, -3e3, 1e4, -3e4)):
        K[:, :, :, c] = 0
        q[:, :, c] = a
    return K, V, q.astype(np.float16)

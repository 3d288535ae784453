/*
 * tkq.h - C ABI of the MI355X (gfx950) low-bit weight GEMV library.
 *
 * The library computes the batch-1 decode product y = dequant(W_q) . x, in
 * which every weight is read once and used for one multiply-add (Whetstone
 * README, "The one fact that shapes everything"), for four weight codings,
 * plus the quantize-and-pack step that produces them and the M >= 64 prefill
 * GEMM over the int4 coding.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument named as a tensor (W, codes, meta, scale, bits, x,
 *   y, X, Y, buf, out, dev_descs, logits, head, token, cand, cand_logits,
 *   scratch, workspace) is a DEVICE pointer owned by the caller
 *   (e.g. a torch tensor's data_ptr()).  The library never allocates, frees or
 *   retains device memory, and keeps no mutable global state apart from a
 *   per-thread copy of the last HIP error code.  Host pointers are named
 *   descs / plan and are read (and, for tkq_gemv_prepare, written) during the
 *   call only.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Every device entry point only enqueues work on it and returns; results
 *   are visible after the caller synchronises that stream.  Device faults
 *   surface at that synchronisation, as usual in HIP.
 * - Arguments are validated on the host BEFORE any HIP call.  A non-zero
 *   return is a negative TKQ_E* status and nothing was enqueued (except for
 *   TKQ_EHIP, which reports a failed launch; see tkq_last_hip_error()).
 * - Tensors are dense, row-major and contiguous; "[N][K/8]" means N rows of
 *   K/8 elements.  All device pointers must be 16-byte aligned.
 * - The content of device buffers (codes, descriptors) is not validated:
 *   codes that the packers never emit decode arithmetically (see each format),
 *   and a descriptor table that does not match its plan is undefined
 *   behaviour.
 * - Non-finite weights passed to a packer are a precondition violation.
 *
 * Weight codings (storage layouts)
 * --------------------------------
 * TKQ_FMT_INT4_G128 (Whetstone README, "What the weights can actually
 *   survive": round-to-nearest int4 in groups of 128, each group with an
 *   fp16 scale and an fp16 zero-point, 4.25 bits/weight):
 *     codes uint32 [N][K/8]  : element 8j+i of a row in bits [4i,4i+4) of word j
 *     meta  uint32 [N][K/128]: fp16 scale in bits [0,16), fp16 zero in [16,32)
 *     w = scale * (q - zero)
 * TKQ_FMT_K5_G128 (TKintegers K5, "What is K5?": one byte per weight holding
 *   five balanced trits, 243 values):
 *     codes uint8 [N][K], scale fp16 [N][K/128]
 *     w = scale * (c - 121); bytes 243..255 are never produced and decode as
 *     c - 121 as well.
 * TKQ_FMT_TERN_G128 (Whetstone README, bytes/token table, "ternary g128"):
 *     codes uint32 [N][K/16]: element 16j+i in bits [2i,2i+2), code = t + 1
 *     scale fp16 [N][K/128];  w = scale * (code - 1); code 3 is never produced
 *     and decodes as +2.
 * TKQ_FMT_BIN (Whetstone README, "Measured hardware facts": {-1,+1} packed as
 *   bits {1,0}):
 *     bits uint32 [N][K/32]  : element 32j+i in bit i of word j, 1 <=> -1
 *     no metadata; x is packed the same way (uint32 [K/32]); y is int32.
 * TKQ_FMT_INT2_G128 (Whetstone README, bytes/token and quality tables, "int2
 *   g128" at 2.25 bits/weight):
 *     codes uint32 [N][K/16] : element 16j+i in bits [2i,2i+2) of word j
 *     meta  uint32 [N][K/128]: as TKQ_FMT_INT4_G128;  w = scale * (q - zero)
 * TKQ_FMT_INT3_G128 (Whetstone README, bytes/token and quality tables, "int3
 *   g128" at 3.25 bits/weight):
 *     codes uint32 [3][N][K/32]: per 128-group g, block b (codes 32b..32b+31)
 *           is three words W0..W2; Wj holds code 10j+f in bits [3f,3f+3) and
 *           code 10j+5+f in bits [16+3f,16+3f+3) (f = 0..4), bit j of code 30
 *           in bit 15 and bit j of code 31 in bit 31.  The group's 12 words
 *           (b0W0, b0W1, b0W2, b1W0, ...) form three 16-byte planes (words
 *           0-3, 4-7, 8-11).  The matrix is stored plane-major: plane p of
 *           group g of row n is at byte p*N*K/8 + n*K/8 + 16g.
 *     meta  uint32 [N][K/128]: as TKQ_FMT_INT4_G128;  w = scale * (q - zero)
 * TKQ_FMT_INT4_HIER_G32 (Whetstone README, bytes/token table "int4 hier-g32"
 *   at 4.28 bits/weight, quantizer table "group 32 with hierarchical scale
 *   metadata", and "Prior art": Q4_K-like sub-scales against an fp16 pair,
 *   with a whole row as the super-block and 4-bit indices):
 *     codes uint32 [N][K/8]  : as TKQ_FMT_INT4_G128
 *     meta  one block of tkq_hier_meta_bytes(N, K) bytes:
 *           bytes [0, N*K/32): byte n*(K/32)+g = sc | mi << 4 for group g
 *                              (columns 32g..32g+31) of row n;
 *           zero bytes up to R = N*K/32 rounded up to a multiple of 16;
 *           uint32 [N] at byte R: fp16 d in bits [0,16), fp16 dmin in
 *                              bits [16,32) of row n.
 *     w = d * sc * q - dmin * mi
 */
#ifndef TKQ_H
#define TKQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TKQ_VERSION 10000 /* major*10000 + minor*100 + patch */

/* ---- status codes ------------------------------------------------------ */
#define TKQ_OK 0
#define TKQ_EINVAL (-1)  /* null pointer, non-positive size, bad count     */
#define TKQ_ESHAPE (-2)  /* K not a multiple of the format's unit, size
                            beyond the supported range                     */
#define TKQ_EALIGN (-3)  /* a device pointer is not 16-byte aligned        */
#define TKQ_EFORMAT (-4) /* unknown format, or mixed formats in one call   */
#define TKQ_EHIP (-5)    /* a HIP call failed: see tkq_last_hip_error()    */
#define TKQ_EPLAN (-6)   /* plan not produced by tkq_gemv_prepare          */

/* ---- weight codings ---------------------------------------------------- */
#define TKQ_FMT_INT4_G128 1
#define TKQ_FMT_K5_G128 2
#define TKQ_FMT_TERN_G128 3
#define TKQ_FMT_BIN 4
#define TKQ_FMT_INT4_HIER_G32 5
#define TKQ_FMT_INT2_G128 6
#define TKQ_FMT_INT3_G128 7

/* Size limits: 1 <= N <= 2^31-1, 32 <= K <= 2^20 (K % 128 == 0 for the
 * group-128 codings and for their GEMVs; K % 32 == 0 for tkq_pack_bin, the
 * int4-hier-g32 coding and their GEMVs), and N*K <= 2^39 weights.  A GEMV
 * additionally needs K <= 32768 (int4 g128, hier-g32, ternary, int2, int3),
 * 16384 (K5) or 262144 (binary). */
#define TKQ_MAX_K (1 << 20)

/* Library version (TKQ_VERSION of the build). */
int tkq_version(void);

/* Static string describing a status code (never NULL). */
const char* tkq_strerror(int status);

/* hipError_t of the last failed HIP call made by this thread (0 if none). */
int tkq_last_hip_error(void);

/* ---- quantize + pack ----------------------------------------------------
 * W is fp32 [N][K] on the device.  Each function writes every output element
 * exactly once; the results are bit-identical to an IEEE fp32 evaluation of
 * the formulas below (true division, rint = round half to even, fp32->fp16
 * round to nearest even).  A scale that rounds to fp16 zero is stored as 1.0
 * (Whetstone README, status list: the fp16 scale that underflowed to zero).
 */

/* int4 g128, asymmetric RTN (Whetstone README, "What the weights can
 * actually survive").  Per row and 128-column group:
 *   lo = min(min w, 0), hi = max(max w, 0), s = fp16((hi - lo) / 15),
 *   z = clamp(rint(-lo / s), 0, 15), q = clamp(rint(w / s) + z, 0, 15).
 * codes: uint32 [N][K/8]; meta: uint32 [N][K/128] = half2 {s, z}.
 * K % 128 == 0. */
int tkq_pack_int4_g128(const float* W, int64_t N, int64_t K, uint32_t* codes,
                       uint32_t* meta, void* stream);

/* K5 byte codes (TKintegers K5, "What is K5?"), symmetric absmax RTN per
 * 128-column group: s = fp16(max|w| / 121), c = clamp(rint(w / s), -121,
 * 121) + 121.  codes: uint8 [N][K]; scale: fp16 bits [N][K/128].
 * K % 128 == 0. */
int tkq_pack_k5(const float* W, int64_t N, int64_t K, uint8_t* codes,
                uint16_t* scale, void* stream);

/* Ternary g128 (Whetstone README, "ternary g128"), absmean RTN per group:
 * s = fp16((|w_0| + |w_1| + ... + |w_127|) / 128) summed in k order in fp32,
 * t = clamp(rint(w / s), -1, 1), code = t + 1.
 * codes: uint32 [N][K/16]; scale: fp16 bits [N][K/128].  K % 128 == 0. */
int tkq_pack_tern_g128(const float* W, int64_t N, int64_t K, uint32_t* codes,
                       uint16_t* scale, void* stream);

/* int2 g128, asymmetric RTN (Whetstone README, "int2 g128"): the int4 g128
 * quantizer with four levels: s = fp16((hi - lo) / 3), z = clamp(rint(-lo /
 * s), 0, 3), q = clamp(rint(w / s) + z, 0, 3).  codes: uint32 [N][K/16];
 * meta: uint32 [N][K/128] = half2 {s, z}.  K % 128 == 0. */
int tkq_pack_int2_g128(const float* W, int64_t N, int64_t K, uint32_t* codes,
                       uint32_t* meta, void* stream);

/* int3 g128, asymmetric RTN (Whetstone README, "int3 g128"): the int4 g128
 * quantizer with eight levels: s = fp16((hi - lo) / 7), z = clamp(rint(-lo /
 * s), 0, 7), q = clamp(rint(w / s) + z, 0, 7).  codes: uint32 [3][N][K/32]
 * in the plane-major layout above; meta: uint32 [N][K/128] = half2 {s, z}.
 * K % 128 == 0. */
int tkq_pack_int3_g128(const float* W, int64_t N, int64_t K, uint32_t* codes,
                       uint32_t* meta, void* stream);

/* Sign bits (Whetstone README, "Measured hardware facts"): bit = 1 exactly
 * when w < 0.  bits: uint32 [N][K/32].  K % 32 == 0.  Also packs x (N = 1). */
int tkq_pack_bin(const float* W, int64_t N, int64_t K, uint32_t* bits,
                 void* stream);

/* int4-hier-g32, RTN at both levels (the pages print no fitting procedure).
 * Per row, for every 32-column group g:
 *   lo = min(min w, 0), hi = max(max w, 0), s_g = (hi - lo) / 15, m_g = -lo;
 * then per row
 *   d = fp16(max_g s_g / 15), dmin = fp16(max_g m_g / 15)  (0 -> 1.0),
 *   sc_g = clamp(rint(s_g / d), 1, 15), mi_g = clamp(rint(m_g / dmin), 0, 15),
 *   q = clamp(rint((w + dmin * mi_g) / (d * sc_g)), 0, 15)
 * (d * sc_g and dmin * mi_g are exact in fp32).  codes: uint32 [N][K/8];
 * meta: tkq_hier_meta_bytes(N, K) bytes (layout above; the padding is
 * written as zeros).  K % 32 == 0; codes and meta 16-byte aligned. */
int tkq_pack_int4_hier_g32(const float* W, int64_t N, int64_t K,
                           uint32_t* codes, uint8_t* meta, void* stream);

/* Bytes of an int4-hier-g32 metadata block for an N x K matrix (host only;
 * -1 if N < 1, K < 32 or K % 32 != 0). */
int64_t tkq_hier_meta_bytes(int64_t N, int64_t K);

/* ---- grouped GEMV -------------------------------------------------------
 * One launch computes any number of independent GEMVs y_i = W_i . x_i that
 * share one coding (e.g. every linear layer read for one decoded token).
 *
 * Float codings: y[n] = sum_k w[n,k] x[k], fp32 accumulation, fp16 output
 * rounded to nearest even; |y - y_exact| <= 2e-3 * sum_k |w[n,k] x[k]|.
 * int4, K5, ternary, int2 and int3: for any finite fp16 x (the code offset
 * is removed exactly before each product, so the rounding error follows
 * |w x|, also on activation channels far larger than their weights).
 * int4-hier-g32: its weight is the difference d sc q - dmin mi of two terms
 * that the coding sums separately over each 32-group (sum q x and sum x),
 * so the error follows (|d sc q| + |dmin mi|) |x|; the bound holds unless
 * activations far larger than the rest meet weights whose two terms nearly
 * cancel.
 * Binary: y[n] = K - 2 * popcount(W[n] XOR x) (Whetstone README, "Measured
 * hardware facts"), exact int32.
 *
 * Usage: fill fmt, N, K, codes, meta, x, y of each host descriptor; call
 * tkq_gemv_prepare (fills the [prepare] fields and the plan); copy the
 * descriptor array to device memory (16-byte aligned); call tkq_gemv with the
 * plan and the device copy, as often as wanted.  Outputs must not overlap
 * each other or any input.
 */
typedef struct tkq_gemv_desc {
  int32_t fmt;           /* TKQ_FMT_*; identical in every descriptor        */
  int32_t N;             /* rows = length of y, >= 1                        */
  int32_t K;             /* columns = length of x, multiple of 128 (of 32
                            for TKQ_FMT_INT4_HIER_G32)                      */
  int32_t work0;         /* [prepare] index of the first row tile           */
  int32_t big_tiles;     /* [prepare] number of large tiles (rows_per_tile
                                      rows each) at the top of the matrix   */
  int32_t rows_per_tile; /* [prepare] rows of a large tile                  */
  int32_t shape;         /* [prepare] lanes-per-row log2 | passes<<4 |
                                      k-slices<<16                          */
  int32_t small_rows;    /* [prepare] rows of a small tile; small tiles
                                      cover the rows below the large ones   */
  const void* codes;     /* packed codes (layout per fmt)                   */
  const void* meta;      /* int4, int3, int2: uint32 half2 [N][K/128]; K5, ternary: fp16
                            [N][K/128]; hier-g32: its metadata block;
                            binary: ignored (may be NULL)                   */
  const void* x;         /* fp16 [K]; binary: uint32 [K/32]                 */
  void* y;               /* fp16 [N]; binary: int32 [N]                     */
} tkq_gemv_desc;         /* 64 bytes */

typedef struct tkq_gemv_plan {
  int32_t fmt;        /* common coding of the descriptors                   */
  int32_t count;      /* number of descriptors                              */
  int64_t tiles;      /* total row tiles = workgroups per launch            */
  int32_t variant;    /* largest pass count: selects the kernel variant
                         (int4: sizes the LDS copy of x, K / 128)          */
  int32_t magic;      /* set by tkq_gemv_prepare                            */
  int64_t reserved;
} tkq_gemv_plan;

/* Host only.  Validates every descriptor (fmt, sizes, non-null and 16-byte
 * aligned pointers, all fmt equal), chooses each GEMV's work decomposition,
 * writes the [prepare] fields of descs[0..count) and fills *plan.
 * Returns TKQ_OK or TKQ_EINVAL / TKQ_ESHAPE / TKQ_EALIGN / TKQ_EFORMAT. */
int tkq_gemv_prepare(tkq_gemv_desc* descs, int32_t count, tkq_gemv_plan* plan);

/* Launches one kernel over plan->tiles workgroups on `stream`.
 * dev_descs: device copy of the prepared descriptors (plan->count of them,
 * 16-byte aligned).  Returns TKQ_OK, TKQ_EINVAL, TKQ_EALIGN, TKQ_EPLAN or
 * TKQ_EHIP. */
int tkq_gemv(const tkq_gemv_plan* plan, const tkq_gemv_desc* dev_descs,
             void* stream);

/* Grouped GEMV plus greedy selection (Whetstone README, status list: the
 * greedy decode path never leaves the GPU; the output projection is the
 * last GEMV of a token).  Computes exactly what tkq_gemv computes, and the
 * index of the largest output of descriptor `target` (0 <= target < count),
 * written to *token (device int32).  The workgroups of the target reduce
 * their outputs in registers as they store them; a second, one-workgroup
 * kernel on the same stream combines the per-tile results.  The comparison
 * is on the stored outputs (fp16 bits for the float codings, -0 equal to +0;
 * int32 for binary); on equal values the smallest index wins; every NaN
 * output (either sign) counts as larger than +inf, so the first NaN wins.
 * scratch: caller-owned device memory of scratch_bytes >= 8 * plan->tiles,
 * 16-byte aligned, any contents (overwritten).  Calls that share a scratch
 * buffer or token must not run concurrently.
 * Returns as tkq_gemv, plus TKQ_EINVAL (target out of range, null token or
 * scratch, scratch too small) and TKQ_EALIGN (token not 4-byte or scratch
 * not 16-byte aligned). */
int tkq_gemv_argmax(const tkq_gemv_plan* plan, const tkq_gemv_desc* dev_descs,
                    int32_t target, int32_t* token, uint64_t* scratch,
                    int64_t scratch_bytes, void* stream);

/* tkq_gemv_argmax without caller scratch, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The per-tile keys go to a fixed array
 * inside the library: TKQ_STATIC_SLOTS 64-bit slots (512 KB) per GPU, held
 * by every GPU the library runs on until the process ends; its address is
 * looked up (hipGetSymbolAddress) on the first call on each device, with the
 * caller's current device, which must be the device of `stream`.  Nothing in
 * the array needs clearing: each launch writes every slot it reads.  No
 * device memory is allocated or freed.  All calls on one GPU share the
 * array, so calls that may overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  Otherwise as
 * tkq_gemv_argmax: returns TKQ_OK, TKQ_EINVAL (target out of range, null
 * token, no usable device), TKQ_ESHAPE (plan->tiles > TKQ_STATIC_SLOTS),
 * TKQ_EALIGN (token not 4-byte aligned), TKQ_EPLAN or TKQ_EHIP. */
#define TKQ_STATIC_SLOTS 65536
int tkq_gemv_argmax_static(const tkq_gemv_plan* plan,
                           const tkq_gemv_desc* dev_descs, int32_t target,
                           int32_t* token, void* stream);

/* Greedy selection with head rescore (Whetstone README, "New in 0.6.0", the
 * head-rescore item: an fp16 copy of the output projection is kept beside
 * the quantized one, and only the logits that decide the token are computed
 * again from that copy).  Run after the quantized output projection has
 * stored its logits (tkq_gemv), on the same stream.
 *   candidates: the k largest stored logits in the order of greedy selection
 *     (the order of tkq_gemv_argmax: -0 equal to +0, every NaN above +inf, on
 *     equal values the smaller row first);
 *   recomputed logit of candidate row r: sum_j head[r][j] * x[j], fp16 x fp16
 *     products (exact in fp32) summed in fp32, so
 *     |l - l_exact| <= gamma_(K-1) * sum_j |head[r][j] x[j]| with
 *     gamma_m = m u / (1 - m u), u = 2^-24 (any summation order);
 *   *token: the candidate whose recomputed logit is largest, in that same
 *     order (NaN above every number, smaller row on ties).
 * logits: fp16 bits [n] (the stored outputs of the quantized projection);
 * head: fp16 bits [n][K], row-major; x: fp16 bits [K] (the projection's
 * input); token: device int32.  cand (device int32 [k]) and cand_logits
 * (device float [k]) are optional (NULL to skip): the candidate rows in
 * greedy order and their recomputed logits.  One workgroup, all
 * intermediate state in LDS: no scratch memory.
 * Limits: 1 <= k <= min(n, TKQ_RESCORE_MAX_K); n < 2^31; K % 8 == 0,
 * K <= TKQ_MAX_K; k * 8 * ceil(ceil(n / 8) / 1024) <= TKQ_RESCORE_CAP (the
 * candidates are collected from k shares of that many logits each: e.g.
 * k <= 107 at n = 151,936, k <= 64 up to n = 262,144).
 * Returns TKQ_OK, TKQ_EINVAL (null logits, head, x or token; n, K or k < 1;
 * k > n), TKQ_ESHAPE (the limits above), TKQ_EALIGN (logits, head or x not
 * 16-byte aligned; token, cand or cand_logits not 4-byte aligned) or
 * TKQ_EHIP. */
#define TKQ_RESCORE_MAX_K 1024
#define TKQ_RESCORE_CAP 16384
int tkq_head_rescore(const uint16_t* logits, int64_t n, const uint16_t* head,
                     const uint16_t* x, int64_t K, int32_t k, int32_t* token,
                     int32_t* cand, float* cand_logits, void* stream);

/* Grouped GEMV plus greedy selection with head rescore over descriptor
 * `target` (the output projection): computes exactly what tkq_gemv computes,
 * and then what tkq_head_rescore computes over the target's stored outputs,
 * with x = the target's x.  The GEMV workgroups of the target store the
 * largest output key of each of their row tiles in `scratch`, so the
 * candidates are found from those keys and the rows of at most k tiles
 * instead of a pass over every output (when ties or large tiles would leave
 * more keys to collect than TKQ_RESCORE_CAP, the selection falls back to the
 * pass over every output; the result is the same).
 * N, K: the target descriptor's N and K (a mismatch is undefined behaviour,
 * like a descriptor table that does not match its plan); head: fp16 bits
 * [N][K], row-major; token, cand, cand_logits, k: as tkq_head_rescore.
 * scratch: caller-owned device memory of scratch_bytes >= 8 * plan->tiles,
 * 16-byte aligned, any contents (overwritten).  Calls that share a scratch
 * buffer or outputs must not run concurrently.
 * Returns as tkq_gemv, plus TKQ_EFORMAT (binary coding: its outputs are
 * int32), TKQ_EINVAL (target out of range; null head, token or scratch;
 * scratch too small; N, K or k < 1; k > N), TKQ_ESHAPE (the limits of
 * tkq_head_rescore for n = N) and TKQ_EALIGN (head or scratch not 16-byte
 * aligned; token, cand or cand_logits not 4-byte aligned). */
int tkq_gemv_argmax_rescore(const tkq_gemv_plan* plan,
                            const tkq_gemv_desc* dev_descs, int32_t target,
                            int64_t N, int64_t K, const uint16_t* head,
                            int32_t k, int32_t* token, int32_t* cand,
                            float* cand_logits, uint64_t* scratch,
                            int64_t scratch_bytes, void* stream);

/* ---- multi-token GEMV (M = 1..16) ----------------------------------------
 * Y_i[m, n] = sum_k X_i[m, k] * w_i[n, k] for M tokens at once over many
 * int4 g128 or int4-hier-g32 matrices in one launch: the regime between
 * batch-1 decode and prefill (Whetstone README, "Prior art": speculative
 * verification and prefill, where several tokens share each weight read).
 * Each weight is read from HBM once and used M times; the products run on
 * the matrix cores from fp16 weights with fp32 accumulation; fp16 output
 * rounded to nearest even.
 * int4 g128: weights s * (q - z) (one rounding);
 *   |Y - Y_exact| <= 2e-3 * sum_k |X[m,k] w[n,k]| entry-wise.
 * int4-hier-g32: weights fma(q, fp16(d sc), -fp16(dmin mi)) in fp16 (three
 *   roundings); |Y - Y_exact| <= 2e-3 * sum_k |X[m,k]| (|d sc q| + |dmin mi|)
 *   entry-wise, while d sc and dmin mi are normal fp16 numbers (any weights
 *   of ordinary magnitude).
 *
 * Descriptors as for tkq_gemv with fmt = TKQ_FMT_INT4_G128 or
 * TKQ_FMT_INT4_HIER_G32 (one coding per call), except
 *   x: fp16 [M][K] (token-major), y: fp16 [M][N] (token-major).
 * tkq_gemm_small_prepare (host only) validates them (K % 128 == 0 for both
 * codings, M*K and M*N below 2^30), fills the [prepare] fields and *plan for
 * this M; a plan from tkq_gemv_prepare is not accepted here, nor the reverse.
 * Returns TKQ_OK, TKQ_EINVAL (null pointers, count or M < 1), TKQ_ESHAPE
 * (M > 16 or sizes), TKQ_EFORMAT (another coding, or codings mixed) or
 * TKQ_EALIGN. */
int tkq_gemm_small_prepare(tkq_gemv_desc* descs, int32_t count, int32_t M,
                           tkq_gemv_plan* plan);

/* Launches the prepared multi-token GEMV on `stream` (dev_descs: device copy
 * of the prepared descriptors, 16-byte aligned).  Returns TKQ_OK,
 * TKQ_EINVAL, TKQ_EALIGN, TKQ_EPLAN or TKQ_EHIP. */
int tkq_gemm_small(const tkq_gemv_plan* plan, const tkq_gemv_desc* dev_descs,
                   void* stream);

/* ---- low-bit KV cache and decode attention ------------------------------
 * (BitDecoding README: 4-bit KV cache codes in groups of 128, K quantized per
 * channel and V per token, head dimension 128, single-query decode.)
 * The cache of one (batch, KV head) is a sequence of pages of 128 tokens,
 * 17408 bytes each:
 *   words [0, 2048)     K codes: token t, channel c in word 16t + c/8,
 *                       bits [4(c%8), 4(c%8)+4)
 *   words [2048, 4096)  V codes: token t, channel c in word 2048 + 16c + t/8,
 *                       bits [4(t%8), 4(t%8)+4)
 *   words [4096, 4224)  K half2 {scale, zero} of channel c (over the page)
 *   words [4224, 4352)  V half2 {scale, zero} of token t (over its channels)
 * value = scale * (code - zero); the quantizer is the int4 g128 one above
 * (lo = min(min, 0), hi = max(max, 0), s = fp16((hi - lo) / 15), integer z).
 * The cache tensor is [B][Hk][T/128][17408 bytes].
 * Shapes: head dimension D = 128, T % 128 == 0, H % Hk == 0; query head h
 * reads KV head h / (H / Hk).  T is the cache's capacity in tokens; the
 * _varlen entry points take per-sequence lengths (BitDecoding README, usage
 * example: every sequence of a batch has its own cached length), so the
 * last page of a sequence may be partly filled. */

/* Bytes of a cache for B x Hk x T tokens (host only; -1 if invalid). */
int64_t tkq_kv_cache_bytes(int32_t B, int32_t Hk, int32_t T);

/* Quantize and page a whole cache.  K, V: fp16 bits [B][T][Hk][D]
 * (token-major), cache: tkq_kv_cache_bytes bytes; all 16-byte aligned.
 * Bit-identical to an IEEE fp32 evaluation of the quantizer.
 * Returns TKQ_OK, TKQ_EINVAL, TKQ_ESHAPE, TKQ_EALIGN or TKQ_EHIP. */
int tkq_kv_pack(const uint16_t* K, const uint16_t* V, int32_t B, int32_t T,
                int32_t Hk, int32_t D, uint32_t* cache, void* stream);

/* tkq_kv_pack for sequences of their own lengths: seqlens is a device int32
 * [B] (4-byte aligned), each value clamped to [0, T].  Tokens t >= seqlens[b]
 * are quantized as zeros (a K group, one channel over a page, spans 0
 * anyway, so its scale and zero-point are those of the valid tokens; such a
 * V token is an all-zero group).  Returns as tkq_kv_pack, plus TKQ_EINVAL
 * for a null seqlens. */
int tkq_kv_pack_varlen(const uint16_t* K, const uint16_t* V,
                       const int32_t* seqlens, int32_t B, int32_t T,
                       int32_t Hk, int32_t D, uint32_t* cache, void* stream);

/* Workspace bytes tkq_kv_decode needs (host only; -1 if invalid). */
int64_t tkq_kv_decode_workspace_bytes(int32_t B, int32_t H, int32_t Hk,
                                      int32_t T);

/* One decode step: out[b,h,:] = softmax(sm_scale * q[b,h,:] . K^T) . V over
 * the T cached tokens of KV head h / (H / Hk), with K and V the dequantized
 * cache.  q, out: fp16 bits [B][H][D].
 * workspace: caller-owned device memory of at least
 * tkq_kv_decode_workspace_bytes.  Its first 4*B*H bytes (rounded up to 16)
 * are arrival counters that must be zero when a call starts, followed by
 * per-split partial results; every completed call leaves its own counters
 * at zero again (and partial results after them).  So: zero-fill the
 * workspace before its first use, and again after a failed call or before a
 * call with a larger B*H than the previous call on it.  Calls that share a
 * workspace must be ordered (one stream).
 * One kernel on `stream`: the workgroups of each (sequence, query-head
 * group) split its pages, and the last of them to finish merges the splits
 * (log-sum-exp) and writes out.
 * Accuracy: both products are held to the GEMV's per-row bound (scores:
 * |ds_t| <= e A_t, A_t = sm_scale sum_c |q_c K_t,c|; output: e sum_t p_t
 * |V_t,c|, e = 2e-3), so per element |out - exact| <= ((1 + e) exp(2 e max_t
 * A_t) - 1) sum_t p_t |V_t,c|.  (The kernels round the query times the K
 * channel scale and the probability times the V token scale to fp16,
 * accumulate in fp32 and round out to fp16.)
 * Returns TKQ_OK, TKQ_EINVAL (null pointers, sm_scale not positive and
 * finite, workspace too small), TKQ_ESHAPE, TKQ_EALIGN or TKQ_EHIP. */
int tkq_kv_decode(const uint16_t* q, const uint32_t* cache, int32_t B,
                  int32_t H, int32_t Hk, int32_t T, int32_t D, float sm_scale,
                  uint16_t* out, float* workspace, int64_t workspace_bytes,
                  void* stream);

/* tkq_kv_decode over the first seqlens[b] tokens of sequence b (device int32
 * [B], 4-byte aligned, each clamped to [0, T]): pages past the length are not
 * read and the tokens past it in the last page take no part; a sequence of
 * length 0 gets out = 0.  Returns as tkq_kv_decode, plus TKQ_EINVAL for a
 * null seqlens. */
int tkq_kv_decode_varlen(const uint16_t* q, const uint32_t* cache,
                         const int32_t* seqlens, int32_t B, int32_t H,
                         int32_t Hk, int32_t T, int32_t D, float sm_scale,
                         uint16_t* out, float* workspace,
                         int64_t workspace_bytes, void* stream);

/* ---- prefill GEMM -------------------------------------------------------
 * Y[m,n] = sum_k X[m,k] * w[n,k] with w the int4 g128 dequantized weights
 * (TKintegers K5, "What is K5?": tiles of low-bit codes are expanded to fp16
 * matrix-core operands with fp32 accumulation).  fp16 output rounded to
 * nearest even; |Y - Y_exact| <= 2e-3 * sum_k |X[m,k] w[n,k]| entry-wise.
 * fmt must be TKQ_FMT_INT4_G128.  X: fp16 bits [M][K]; Y: fp16 bits [M][N];
 * codes, meta as produced by tkq_pack_int4_g128.  Any M >= 1; tuned for
 * M >= 64 (decode, M = 1, belongs to tkq_gemv).  K % 128 == 0.
 * workspace (optional, may be NULL with workspace_bytes 0): caller-owned
 * device memory, 16-byte aligned, not overlapping any other argument.  When
 * it holds at least 2*M*N floats the library may split K over workgroups,
 * writing fp32 partial products there and summing them in a second kernel
 * on the same stream; its contents are undefined afterwards.  Calls that
 * share one workspace must be ordered (same stream). */
int tkq_gemm_prefill(int32_t fmt, int64_t M, int64_t N, int64_t K,
                     const uint32_t* codes, const uint32_t* meta,
                     const uint16_t* X, uint16_t* Y, float* workspace,
                     int64_t workspace_bytes, void* stream);

/* ---- bandwidth probe ----------------------------------------------------
 * Reads `bytes` bytes of `buf` once with the same 16-byte non-temporal loads
 * the GEMV uses and writes their XOR into out[0..3] (uint32 x 4), so that the
 * read cannot be elided.  bytes % 16 == 0, bytes >= 16.  A reference for the
 * achievable HBM read rate; not part of the GEMV. */
int tkq_read_probe(const void* buf, int64_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TKQ_H */

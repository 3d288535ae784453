// Multi-token GEMV over int4 g128 or int4-hier-g32 weights for gfx950:
// Y[m, n] = sum_k X[m, k] * w[n, k] for M = 1..16 tokens at once
// (speculative verification, short prefill: Whetstone README, "Prior art",
// where several tokens share every weight read; the timing table's 16-token
// pass).
//
// Every weight is still read from HBM once, but it is used M times, so at
// M = 16 the arithmetic (~60 flop per byte of int4) is beyond the vector ALUs
// at full bandwidth; the products run on the matrix cores:
//
//  * One wave owns 16 weight rows; a workgroup (4 waves) owns 64 rows of one
//    matrix, and a grouped launch concatenates the tiles of many matrices
//    (a scalar binary search finds a workgroup's matrix, as in the GEMV).
//  * Per 128-column quantization group, lane l loads one 16-byte chunk: row
//    l % 16, columns 32 (l / 16) .. +31 of the group.  These are exactly the
//    A operands of four v_mfma_f32_16x16x32_f16 (lane l supplies row l % 16
//    and the k-block l / 16), so the weights go from HBM to the matrix cores
//    through registers only.  The chunk is unpacked with the fp16 magic
//    number (1024 + m * code), shifted by the zero point (exact small
//    integers) and scaled (one fp16 rounding of s * (q - z)).
//  * int4-hier-g32 (Whetstone README, quantizer table, "group 32 with
//    hierarchical scale metadata"): the 16-byte chunk is exactly one
//    32-group, and a group's index byte sits where the g128 coding keeps a
//    group's half2, 4 bytes per 128 columns (lane c takes byte c).  The
//    lane forms the group's step S = fp16(d sc) and offset O = fp16(dmin mi)
//    with one packed fp16 multiply of (sc, mi) by the row's (d, dmin), and
//    each weight is fma(q, S, -O) in fp16: three roundings, so the error of
//    a weight is below 2^-10 (|d sc q| + |dmin mi|).
//  * The tokens' x slices are staged through LDS, KC columns per round (512
//    for M > 8: fewer registers and more waves, +3-5 % at M = 16; 1024 for
//    M <= 8, where longer rounds measured equal or better), in
//    the k order the unpack produces (0, 4, 1, 5, 2, 6, 3, 7 within each 8),
//    and read as the B operands (lane l: token l % 16, k-block l / 16).
//    Lanes of tokens >= M read LDS rows zeroed once per workgroup, so the
//    B-operand reads need no condition (one without a condition lets the
//    compiler issue them ahead of their MFMAs).
//  * The codes of round i + 1 are loaded into a second register buffer
//    while round i is computed, so every wave keeps its next KC / 2 bytes
//    per row in flight.
//  * fp32 accumulation; Y rounded to fp16 (nearest even) on store.
#include "device_common.h"
#include "kernels.h"

namespace tkq {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 hv2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kTileRows = kSmallTileRows;  // 16 rows per wave
// Columns of X staged per round: 512 for M > kKcSplit, 1024 otherwise.
constexpr int kKcBigM = 512, kKcSmallM = 1024, kKcSplit = 8;
template <int KC>
constexpr int lds_row() { return KC + 8; }  // halves per staged token row (16 bytes of padding)
constexpr int NACC = 1;  // accumulators (MFMA dependency chains; 2-4 measured slower)
constexpr uint32_t kMagic = 0x64006400u;

__device__ __forceinline__ uint32_t in_sgpr(uint32_t c) {
  uint32_t r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "i"(c));
  return r;
}
__device__ __forceinline__ uint32_t in_vgpr(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}
__device__ __forceinline__ hv2 h2(uint32_t u) { return __builtin_bit_cast(hv2, u); }
__device__ __forceinline__ uint32_t u32h(hv2 h) { return __builtin_bit_cast(uint32_t, h); }

// One code word (8 nibbles, natural order) -> 8 fp16 weights s * (q - z) in
// the order (0, 4, 1, 5, 2, 6, 3, 7).
__device__ __forceinline__ half8 dequant_word(uint32_t w, uint32_t m0, uint32_t m1, uint32_t magic, hv2 nz1,
                                              hv2 nz16, hv2 s) {
  const hv2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t t = w >> 8;
  const hv2 a = (h2((w & m0) | magic) + nz1) * s;                    // (q0, q4)
  const hv2 b = (h2((w & m1) | magic) * sixteenth + nz16) * s;       // (q1, q5)
  const hv2 c = (h2((t & m0) | magic) + nz1) * s;                    // (q2, q6)
  const hv2 d = (h2((t & m1) | magic) * sixteenth + nz16) * s;       // (q3, q7)
  u32x4 v = {u32h(a), u32h(b), u32h(c), u32h(d)};
  return __builtin_bit_cast(half8, v);
}

// One code word -> 8 fp16 weights fma(q, S, -O) (int4-hier-g32) in the
// order (0, 4, 1, 5, 2, 6, 3, 7); so = (S, S), no = (-O, -O).  The codes
// themselves come out exact: 1024 + q - 1024, (1024 + 16 q) / 16 - 64.
__device__ __forceinline__ half8 dequant_word_hier(uint32_t w, uint32_t m0, uint32_t m1, uint32_t magic, hv2 so,
                                                   hv2 no) {
  const hv2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const hv2 n1024 = {(_Float16)(-1024.0f), (_Float16)(-1024.0f)};
  const hv2 n64 = {(_Float16)(-64.0f), (_Float16)(-64.0f)};
  const uint32_t t = w >> 8;
  const hv2 a = __builtin_elementwise_fma(h2((w & m0) | magic) + n1024, so, no);
  const hv2 b = __builtin_elementwise_fma(__builtin_elementwise_fma(h2((w & m1) | magic), sixteenth, n64), so, no);
  const hv2 c = __builtin_elementwise_fma(h2((t & m0) | magic) + n1024, so, no);
  const hv2 d = __builtin_elementwise_fma(__builtin_elementwise_fma(h2((t & m1) | magic), sixteenth, n64), so, no);
  u32x4 v = {u32h(a), u32h(b), u32h(c), u32h(d)};
  return __builtin_bit_cast(half8, v);
}

template <int KC>
struct CodeBuf {
  static constexpr int GR = KC / 128;  // quantization groups per round
  u32x4 q[GR];
  uint32_t m[GR];
};

struct SmallTile {
  __amdgpu_buffer_rsrc_t codes, meta, x;
  uint32_t lrow, row_bytes, meta_row;
  int K, M, c, r;
  hv2 dd;  // int4-hier-g32: the lane's row pair (d, dmin)
};

// Groups at or past K load from an offset beyond the buffer (zeros, no
// memory access): the loads stay unconditional, so the compiler can count
// them and wait for exactly the ones a round consumes, not for the next
// round's prefetch too.
constexpr uint32_t kFar = 0x80000000u;
// PRIO: the wave raises its priority while it issues a round's loads, so
// they are not queued behind other waves' unpack and MFMA work (M > 8:
// +2 % on the 0.5B and 7B sweeps at M = 16; at M = 2 it cost 4 %).
template <int KC, bool PRIO>
__device__ __forceinline__ void load_round(const SmallTile& t, int kc, CodeBuf<KC>& b) {
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int g = 0; g < KC / 128; ++g) {
    const bool ok = kc + 128 * g < t.K;  // uniform
    b.q[g] = load16_nt(t.codes, ok ? t.lrow * t.row_bytes + (uint32_t)(kc + 128 * g) / 2u + 16u * t.c : kFar);
    b.m[g] = load4(t.meta, ok ? t.lrow * t.meta_row + (uint32_t)((kc / 128 + g) * 4) : kFar);
  }
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
}

// Stage X[0..M)[kc, kc + KC) into LDS in the unpack's k order.  Thread i
// takes the 8-column unit i % U (U = KC / 8 units per token row) of token
// rows i / U + P j, j < SB (P = token rows per pass of the workgroup), so
// one batch covers every row a variant takes (KC = 512: 4 x 4 = 16 rows;
// KC = 1024: 2 x 4 = 8 rows) with no division.  Each thread issues its SB
// loads before writing any of them (one memory round trip per round); units
// past the round's end or rows past M read beyond the buffer (zeros) and
// are not written.
constexpr int SB = 4;
template <int KC>
__device__ __forceinline__ void stage_x(const SmallTile& t, int kc, _Float16* xs) {
  constexpr int kLdsRow = lds_row<KC>();
  constexpr int U = KC / 8;
  constexpr int P = 64 * kWaves / U;
  static_assert(P * U == 64 * kWaves, "a pass covers whole token rows");
  static_assert(P * SB >= (KC == kKcSmallM ? kKcSplit : kSmallMaxM), "one batch covers every token row");
  const int units = min(KC, t.K - kc) / 8;
  const int e = (int)threadIdx.x % U, m0 = (int)threadIdx.x / U;
  u32x4 v[SB];
#pragma unroll
  for (int j = 0; j < SB; ++j) {
    const int m = m0 + P * j;
    const bool ok = m < t.M && e < units;
    v[j] = load16(t.x, ok ? (uint32_t)(m * t.K + kc + 8 * e) * 2u : kFar);
  }
#pragma unroll
  for (int j = 0; j < SB; ++j) {
    const int m = m0 + P * j;
    if (m < t.M && e < units) {
      u32x4 p;
      p[0] = __builtin_amdgcn_perm(v[j][2], v[j][0], 0x05040100u);  // (x0, x4)
      p[1] = __builtin_amdgcn_perm(v[j][2], v[j][0], 0x07060302u);  // (x1, x5)
      p[2] = __builtin_amdgcn_perm(v[j][3], v[j][1], 0x05040100u);  // (x2, x6)
      p[3] = __builtin_amdgcn_perm(v[j][3], v[j][1], 0x07060302u);  // (x3, x7)
      *reinterpret_cast<u32x4*>(&xs[m * kLdsRow + 8 * e]) = p;
    }
  }
}

template <int KC, bool HIER>
__device__ __forceinline__ void compute_round(const SmallTile& t, int kc, const CodeBuf<KC>& b, const _Float16* xs,
                                              uint32_t m0, uint32_t m1, uint32_t magic, f32x4 (&acc)[NACC]) {
  constexpr int kLdsRow = lds_row<KC>();
  const int ng = min(KC, t.K - kc) / 128;
#pragma unroll
  for (int g = 0; g < KC / 128; ++g) {
    if (g < ng) {
      hv2 s, nz1, nz16 = {};
      if constexpr (HIER) {
        // (1024 + sc, 1024 + mi) from the lane's index byte, then (sc, mi) exactly
        const uint32_t ix = b.m[g] >> (8 * t.c);
        const hv2 scmi = h2((ix & 0xFu) | ((ix & 0xF0u) << 12) | magic) - h2(magic);
        const hv2 so = scmi * t.dd;  // (S, O), one rounding each
        s = (hv2){so[0], so[0]};
        nz1 = (hv2){-so[1], -so[1]};
      } else {
        s = (hv2){h2(b.m[g])[0], h2(b.m[g])[0]};
        const _Float16 z = h2(b.m[g])[1];
        nz1 = (hv2){(_Float16)(-1024.0f) - z, (_Float16)(-1024.0f) - z};
        nz16 = (hv2){(_Float16)(-64.0f) - z, (_Float16)(-64.0f) - z};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half8 a;
        if constexpr (HIER) a = dequant_word_hier(b.q[g][j], m0, m1, magic, s, nz1);
        else a = dequant_word(b.q[g][j], m0, m1, magic, nz1, nz16, s);
        // token rows past M read the zeros written at the start of the kernel
        const half8 xb = *reinterpret_cast<const half8*>(&xs[t.r * kLdsRow + 128 * g + 32 * t.c + 8 * j]);
        acc[j % NACC] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, xb, acc[j % NACC], 0, 0, 0);
      }
    }
  }
}

template <int KC, bool PRIO, bool HIER>
__global__ __launch_bounds__(256) void small_m_kernel(const tkq_gemv_desc* __restrict__ descs, int count, int M) {
  __shared__ __attribute__((aligned(16))) _Float16 xs[16 * lds_row<KC>()];

  const int tile = blockIdx.x;
  // The workgroup's matrix: the last descriptor with work0 <= tile (work0
  // strictly increases).  A 16-way search: each step reads 15 evenly spaced
  // work0 values at once (independent scalar loads, indexes clamped rather
  // than guarded so that none waits for another), so a sweep of up to 256
  // matrices takes two memory round trips instead of eight.  Invariant:
  // work0[lo] <= tile < work0[hi] (hi = count: past the end).  (The
  // batch-1 GEMV keeps its binary search: there the 16-way form measured
  // 0.5-3 % slower, its tiles being long enough to hide the search.)
  int lo = 0, hi = count;
  while (hi - lo > 1) {
    const int step = (hi - lo + 15) >> 4;
    int w[15];
#pragma unroll
    for (int p = 0; p < 15; ++p) w[p] = descs[min(lo + (p + 1) * step, hi - 1)].work0;
    int next = lo;
#pragma unroll
    for (int p = 0; p < 15; ++p)
      if (w[p] <= tile) next = max(next, min(lo + (p + 1) * step, hi - 1));
    hi = min(hi, next + step);
    lo = next;
  }
  const tkq_gemv_desc* d = descs + lo;
  const int N = d->N, K = d->K;
  const int row0 = (tile - d->work0) * kTileRows;
  const int nrows = min(kTileRows, N - row0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  SmallTile t;
  t.r = lane & 15;
  t.c = lane >> 4;
  t.K = K;
  t.M = M;
  t.lrow = (uint32_t)(wave * 16 + t.r);
  t.row_bytes = (uint32_t)K / 2u;
  t.meta_row = (uint32_t)(K / 128) * 4u;
  t.codes = make_rsrc((const char*)d->codes + (size_t)row0 * t.row_bytes, (uint32_t)nrows * t.row_bytes);
  t.meta = make_rsrc((const char*)d->meta + (size_t)row0 * t.meta_row, (uint32_t)nrows * t.meta_row);
  t.x = make_rsrc(d->x, (uint32_t)M * (uint32_t)K * 2u);
  const uint32_t m0 = in_sgpr(0x000F000Fu), m1 = in_sgpr(0x00F000F0u), magic = in_vgpr(kMagic);
  if constexpr (HIER) {  // rows past N read beyond the buffer: zeros
    const __amdgpu_buffer_rsrc_t rm =
        make_rsrc((const char*)d->meta + hier_row_offset(N, K) + (size_t)row0 * 4u, (uint32_t)nrows * 4u);
    t.dd = h2(load4(rm, t.lrow * 4u));
  }

  f32x4 acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  CodeBuf<KC> a, b;
  load_round<KC, PRIO>(t, 0, a);
  // Token rows M..15 of xs are never staged: zero them once, so that the
  // lanes of tokens past M read zeros unconditionally (the first barrier
  // below orders these writes before any read).
  for (int i = threadIdx.x; i < (kSmallMaxM - M) * lds_row<KC>() / 8; i += 64 * kWaves)
    *reinterpret_cast<u32x4*>(&xs[M * lds_row<KC>() + 8 * i]) = (u32x4){0u, 0u, 0u, 0u};
  for (int kc = 0; kc < K; kc += 2 * KC) {
    __syncthreads();  // the previous round's reads of xs are done
    stage_x<KC>(t, kc, xs);
    __syncthreads();
    load_round<KC, PRIO>(t, kc + KC, b);  // past K: no memory access
    compute_round<KC, HIER>(t, kc, a, xs, m0, m1, magic, acc);
    if (kc + KC >= K) break;
    __syncthreads();
    stage_x<KC>(t, kc + KC, xs);
    __syncthreads();
    load_round<KC, PRIO>(t, kc + 2 * KC, a);
    compute_round<KC, HIER>(t, kc + KC, b, xs, m0, m1, magic, acc);
  }

  // lane l holds Y rows 4 (l / 16) + i of the wave's block for token l % 16
#pragma unroll
  for (int i = 1; i < NACC; ++i) acc[0] += acc[i];
  if (t.r < M) {
    const __amdgpu_buffer_rsrc_t y = make_rsrc(d->y, (uint32_t)M * (uint32_t)N * 2u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = row0 + wave * 16 + 4 * t.c + i;
      if (n < N) store2(y, (uint32_t)(t.r * N + n) * 2u, half_bits(acc[0][i]));
    }
  }
}

template <bool HIER>
void launch_small_m_fmt(const tkq_gemv_desc* dev_descs, int count, int64_t tiles, int M, hipStream_t stream) {
  if (M > kKcSplit)
    hipLaunchKernelGGL((small_m_kernel<kKcBigM, true, HIER>), dim3((uint32_t)tiles), dim3(64 * kWaves), 0, stream,
                       dev_descs, count, M);
  else
    hipLaunchKernelGGL((small_m_kernel<kKcSmallM, false, HIER>), dim3((uint32_t)tiles), dim3(64 * kWaves), 0,
                       stream, dev_descs, count, M);
}

}  // namespace

hipError_t launch_small_m(const tkq_gemv_desc* dev_descs, int count, int64_t tiles, int M, bool hier,
                          hipStream_t stream) {
  if (hier) launch_small_m_fmt<true>(dev_descs, count, tiles, M, stream);
  else launch_small_m_fmt<false>(dev_descs, count, tiles, M, stream);
  return hipGetLastError();
}

}  // namespace tkq

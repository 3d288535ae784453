// Greedy selection with head rescore (Whetstone README, "New in 0.6.0", the
// head-rescore item: an fp16 copy of the output projection is kept next to
// the quantized one, and only the logits that decide the token are computed
// again from it).  The candidates are the k largest stored logits in the
// order of greedy selection; each is recomputed from its fp16 head row, and
// the token is the candidate whose recomputed logit is largest.
//
// One workgroup of 1024 threads, no memory beyond LDS:
//  1. every thread takes the largest 16-bit value key over its share of the
//     stored logits (16-byte chunks t, t + 1024, t + 2048, ...), two logits
//     per packed 16-bit instruction;
//  2. tau = the k-th largest share maximum as a 64-bit key (value, then the
//     smaller row): two 256-bin LDS histograms of the share maxima give its
//     value v; when more shares than needed have maximum v, those shares are
//     read again for their first row of value v.  k logits have keys >= tau,
//     so all of the k largest do too, and exactly k shares can hold keys >=
//     tau (every other share's maximum is below it);
//  3. those k shares are read again and every key >= tau is collected in LDS
//     (at most k shares of R chunks of 8 logits);
//  4. the k largest collected keys, in greedy order, are the candidates (a
//     rank count for small collections, else a bitonic sort);
//  5. each candidate's logit is recomputed in fp32 from its fp16 head row and
//     x: fp16 x fp16 products are exact in fp32, so only the fp32 sums round;
//  6. the token is the candidate with the largest recomputed logit.
#include <atomic>

#include "device_common.h"
#include "kernels.h"

namespace tkq {

namespace {

constexpr int kThreads = 1024;
constexpr int kInFlight = 16;    // 16-byte loads a thread issues before using any
constexpr int kRankMax = 256;    // collections up to this size are ranked by counting
constexpr int kBatch = 4;        // chunks (or tile keys) per thread in flight in the collection passes
constexpr uint32_t kFar = 0x80000000u;  // buffer offset past every range: loads return 0, no access
constexpr int kWl = 2 * kThreads;  // worklist entries (uint32, in the candidate array until step 4)

// 16-bit order key of a stored fp16 logit: larger value -> larger key; -0
// counts as +0 and every NaN (either sign, any payload) above +inf.  At least
// 0x03FF for every value, so 0 can mark "empty".
__device__ __forceinline__ uint32_t ord_f16(uint32_t bits) {
  bits &= 0xFFFFu;
  if (bits == 0x8000u) bits = 0u;
  uint32_t ord = (bits & 0x8000u) ? (~bits & 0xFFFFu) : (bits | 0x8000u);
  if ((bits & 0x7FFFu) > 0x7C00u) ord = 0xFFFFu;
  return ord;
}
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// ord_f16 of the two logits in a word, before its two fixes: -0 gives 0x7FFF
// (the key of +0 less one) and NaNs keep their payload order (a +NaN lands
// above 0xFC00 = +inf, a -NaN below 0x03FF = -inf).  Both are repaired on a
// share's maximum and minimum (share_value).
__device__ __forceinline__ u16x2 ord2_raw(uint32_t w) {
  const uint32_t s = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, w) >> (i16x2){15, 15});
  return __builtin_bit_cast(u16x2, w ^ (s | 0x80008000u));
}
// The largest ord_f16 of a set of logits from the max and min of their raw
// keys (0 when the set is empty: max 0, min 0xFFFF).  -0 is the largest value
// exactly when the maximum is 0x7FFF, which becomes +0's key; any NaN makes
// the maximum NaN.
__device__ __forceinline__ uint32_t share_value(uint32_t hi, uint32_t lo) {
  if (hi > 0xFC00u || lo < 0x03FFu) return 0xFFFFu;
  return hi == 0x7FFFu ? 0x8000u : hi;
}

// Order key of a stored logit: the value key, then the smaller row larger.
// Never 0 for a row < 2^32 - 1.
__device__ __forceinline__ uint64_t key_f16(uint32_t bits, uint32_t row) {
  return ((uint64_t)ord_f16(bits) << 32) | (uint64_t)(0xFFFFFFFFu - row);
}
// The same order on fp32 values (the recomputed logits).
__device__ __forceinline__ uint64_t key_f32(float v, uint32_t row) {
  uint32_t b = u32(v);
  if (b == 0x80000000u) b = 0u;
  uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) ord = 0xFFFFFFFFu;
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - row);
}
__device__ __forceinline__ uint32_t key_row(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)key; }

// Keys of the 8 logits of a full chunk v (rows r0 .. r0 + 7).
__device__ __forceinline__ void full_keys(u32x4 v, uint32_t r0, uint64_t kk[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) kk[e] = key_f16((e & 1) ? (v[e >> 1] >> 16) : v[e >> 1], r0 + e);
}
// Keys of logits r0 .. r1 - 1 (up to 8; 0 for the rest), one 2-byte load each.
__device__ __forceinline__ void part_keys(__amdgpu_buffer_rsrc_t rs, uint32_t r0, uint32_t r1, uint64_t kk[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) kk[e] = r0 + e < r1 ? key_f16(load2(rs, (r0 + e) * 2u), r0 + e) : 0;
}
// The largest value key (ord_f16) of a full chunk's 8 logits, two per packed
// instruction: a chunk below a threshold value needs no 64-bit keys.
__device__ __forceinline__ uint32_t chunk_value(u32x4 v) {
  u16x2 vmax = {0, 0}, vmin = {0xFFFF, 0xFFFF};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const u16x2 o = ord2_raw(v[w]);
    vmax = __builtin_elementwise_max(vmax, o);
    vmin = __builtin_elementwise_min(vmin, o);
  }
  return share_value(max((uint32_t)vmax.x, (uint32_t)vmax.y), min((uint32_t)vmin.x, (uint32_t)vmin.y));
}

// Sorts s[0, P) into descending order (P a power of two, <= every thread's
// loop bound); every thread of the workgroup must call it.
__device__ void bitonic_desc(uint64_t* s, int P) {
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < P / 2; i += kThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const uint64_t a = s[lo], b = s[hi];
        const bool desc = (lo & size) == 0;
        if ((a < b) == desc) {
          s[lo] = b;
          s[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// Whole-wave reductions without the LDS pipe: DPP quad and mirror steps within
// rows of 16 lanes, then gfx950's permlane swaps across rows (with the value
// in both operands the two results hold each lane's own value and that of
// lane ^ 16 or ^ 32).  The result is in every lane.
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float wave_sum(float v) {
  v += f32(dppu<kQuadSwap1>(u32(v)));
  v += f32(dppu<kQuadSwap2>(u32(v)));
  v += f32(dppu<kRowHalfMirror>(u32(v)));
  v += f32(dppu<kRowMirror>(u32(v)));
  auto r = __builtin_amdgcn_permlane16_swap(u32(v), u32(v), false, false);
  v = f32(r[0]) + f32(r[1]);
  r = __builtin_amdgcn_permlane32_swap(u32(v), u32(v), false, false);
  return f32(r[0]) + f32(r[1]);
}
template <int CTRL>
__device__ __forceinline__ uint64_t max_dpp64(uint64_t v) {
  const uint64_t o = ((uint64_t)dppu<CTRL>((uint32_t)(v >> 32)) << 32) | dppu<CTRL>((uint32_t)v);
  return o > v ? o : v;
}
__device__ __forceinline__ uint64_t max_swap64(uint64_t v, bool wide) {
  const uint32_t h = (uint32_t)(v >> 32), l = (uint32_t)v;
  const auto rh = wide ? __builtin_amdgcn_permlane32_swap(h, h, false, false)
                       : __builtin_amdgcn_permlane16_swap(h, h, false, false);
  const auto rl = wide ? __builtin_amdgcn_permlane32_swap(l, l, false, false)
                       : __builtin_amdgcn_permlane16_swap(l, l, false, false);
  const uint64_t a = ((uint64_t)rh[0] << 32) | rl[0], b = ((uint64_t)rh[1] << 32) | rl[1];
  return a > b ? a : b;
}
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
  v = max_dpp64<kQuadSwap1>(v);
  v = max_dpp64<kQuadSwap2>(v);
  v = max_dpp64<kRowHalfMirror>(v);
  v = max_dpp64<kRowMirror>(v);
  return max_swap64(max_swap64(v, false), true);
}

// Wave 0: the largest bin b of hist[256] whose suffix count S(b) (bins >= b)
// reaches `need`, and S(b + 1); need >= 1 and S(0) >= need.  Lane l holds
// bins 255 - 4l .. 252 - 4l (from the top down), so an inclusive prefix sum
// over the lanes (DPP row shifts, then row broadcasts) gives S at each
// lane's lowest bin, and the first lane that reaches `need` holds b.
__device__ __forceinline__ void suffix_select(const uint32_t* hist, uint32_t need, uint32_t* bin,
                                              uint32_t* above) {
  const int lane = threadIdx.x & 63;
  const u32x4 q = *reinterpret_cast<const u32x4*>(hist + 252 - 4 * lane);
  const uint32_t h[4] = {q[3], q[2], q[1], q[0]};  // bins 255 - 4l - i
  const uint32_t sum = h[0] + h[1] + h[2] + h[3];
  uint32_t p = sum;
  p += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)p, 0x111, 0xF, 0xF, false);  // row_shr:1
  p += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)p, 0x112, 0xF, 0xF, false);  // row_shr:2
  p += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)p, 0x114, 0xF, 0xF, false);  // row_shr:4
  p += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)p, 0x118, 0xF, 0xF, false);  // row_shr:8
  p += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)p, kRowBcast15, 0xA, 0xF, false);
  p += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)p, kRowBcast31, 0xC, 0xF, false);
  const uint64_t reached = __ballot(p >= need);
  const int first = __builtin_ctzll(reached);
  if (lane == first) {
    uint32_t cum = p - sum;  // S(256 - 4 lane): the bins above this lane's
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (cum + h[i] >= need) {
        *bin = 255u - 4u * (uint32_t)lane - (uint32_t)i;
        *above = cum;
        break;
      }
      cum += h[i];
    }
  }
}

// Workgroup state of the selection (besides the two dynamic LDS arrays).
struct Lds {
  alignas(16) uint32_t hist1[256], hist2[256];  // read 16 bytes at a time by suffix_select
  uint32_t count, nwin, ntie, bin1, above1, bin2, above2, over, nwl;
  unsigned long long tau;
  int32_t winners[kThreads];
  float exact[TKQ_RESCORE_MAX_K];
  unsigned long long wave_best[kThreads / 64];
};

// Steps 1-3 from the stored logits alone: coll[0, S.count) receives every key
// >= tau (a superset of the k largest), at most k * 8 * R of them.
__device__ __forceinline__ void collect_shares(Lds& S, uint64_t* cands, uint64_t* coll, const uint16_t* logits, int64_t n, int k) {
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int64_t nchunks = (n + 7) / 8, nfull = n / 8;
  const int64_t R = (nchunks + kThreads - 1) / kThreads;  // chunks per share
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(logits, (uint32_t)(n * 2));
  if (t < 256) S.hist1[t] = S.hist2[t] = 0u;
  if (t == 0) S.count = S.nwin = S.ntie = 0u;

  // 1. this thread's share maximum value.  Every round but the last holds a
  // full chunk for every thread; the last one may hold a full, a ragged or no
  // chunk.
  u16x2 vmax = {0, 0}, vmin = {0xFFFF, 0xFFFF};
  const int64_t Rfull = R - 1;
  for (int64_t r0 = 0; r0 < Rfull; r0 += kInFlight) {
    u32x4 v[kInFlight];
    // all loads in one block (one in a branch of its own each made the
    // compiler wait for every earlier load first); past Rfull they read zeros
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      v[u] = load16(rs, r0 + u < Rfull ? (uint32_t)((t + (r0 + u) * kThreads) * 16) : kFar);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      if (r0 + u < Rfull) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const u16x2 o = ord2_raw(v[u][w]);
          vmax = __builtin_elementwise_max(vmax, o);
          vmin = __builtin_elementwise_min(vmin, o);
        }
      }
    }
  }
  const int64_t clast = t + Rfull * kThreads;
  if (clast < nfull) {
    const u32x4 v = load16(rs, (uint32_t)(clast * 16));
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u16x2 o = ord2_raw(v[w]);
      vmax = __builtin_elementwise_max(vmax, o);
      vmin = __builtin_elementwise_min(vmin, o);
    }
  }
  uint32_t M = share_value(max((uint32_t)vmax.x, (uint32_t)vmax.y), min((uint32_t)vmin.x, (uint32_t)vmin.y));
  if (clast >= nfull && clast < nchunks)  // the ragged last chunk
    for (int64_t i = 8 * clast; i < n; ++i) M = max(M, ord_f16(load2(rs, (uint32_t)(i * 2))));
  __syncthreads();

  // 2. tau = the k-th largest share maximum key
  if (M) atomicAdd(&S.hist1[M >> 8], 1u);
  __syncthreads();
  if (min(nchunks, (int64_t)kThreads) <= k) {  // at most k non-empty shares (t < nchunks): take them all
    if (t == 0) S.bin1 = 0xFFFFFFFFu;
  } else if (wave == 0) {
    suffix_select(S.hist1, (uint32_t)k, &S.bin1, &S.above1);
  }
  __syncthreads();
  uint64_t tau = 1;  // every real key is >= 1
  bool winner = M != 0;
  if (S.bin1 != 0xFFFFFFFFu) {
    if (M && (M >> 8) == S.bin1) atomicAdd(&S.hist2[M & 0xFFu], 1u);
    __syncthreads();
    if (wave == 0) suffix_select(S.hist2, (uint32_t)k - S.above1, &S.bin2, &S.above2);
    __syncthreads();
    const uint32_t v16 = (S.bin1 << 8) | S.bin2;
    const uint32_t m = (uint32_t)k - S.above1 - S.above2;  // shares of maximum v16 to take (>= 1)
    winner = M > v16;
    if (S.hist2[S.bin2] == m) {
      // exactly m shares have maximum v16: all of them are winners, and the
      // keys of value >= v16 lie in the k winners' shares only
      tau = (uint64_t)v16 << 32;
      winner = M >= v16;
    } else {
      // more: each tied share's first row of value v16 decides.  The tied
      // shares (listed in `S.winners`) are read again, their first keys of
      // value v16 max-reduced into `cands`; both are free until later steps.
      uint32_t my = 0;
      if (M == v16) {
        my = atomicAdd(&S.ntie, 1u);
        S.winners[my] = t;
        cands[my] = 0;
      }
      __syncthreads();
      const int nt = (int)S.ntie;
      for (int64_t p0 = 0; p0 < (int64_t)nt * R; p0 += kBatch * kThreads) {
        u32x4 v[kBatch];
        int64_t c[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int64_t p = p0 + u * kThreads + t, pp = p < (int64_t)nt * R ? p : 0;
          c[u] = S.winners[pp / R] + (pp % R) * kThreads;
          if (p >= (int64_t)nt * R) c[u] = nchunks;
          v[u] = load16(rs, c[u] < nfull ? (uint32_t)(c[u] * 16) : kFar);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (c[u] >= nchunks) continue;
          uint64_t kk[8];
          if (c[u] < nfull) {
            if (chunk_value(v[u]) < v16) continue;
            full_keys(v[u], (uint32_t)(8 * c[u]), kk);
          } else {
            part_keys(rs, (uint32_t)(8 * c[u]), (uint32_t)n, kk);
          }
          uint64_t f = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) f = (kk[e] >> 32) == v16 && kk[e] > f ? kk[e] : f;
          const int64_t p = p0 + u * kThreads + t;
          if (f) atomicMax(reinterpret_cast<unsigned long long*>(&cands[p / R]), (unsigned long long)f);
        }
      }
      __syncthreads();
      if (M == v16) {
        const uint64_t mine = cands[my];
        uint32_t rank = 0;
        for (int j = 0; j < nt; ++j) rank += cands[j] > mine;
        if (rank == m - 1) S.tau = mine;
        winner = rank < m;
      }
      __syncthreads();
      tau = S.tau;
    }
  }
  if (winner) S.winners[atomicAdd(&S.nwin, 1u)] = t;
  __syncthreads();
  const int W = (int)S.nwin;  // k, or every non-empty share when there are at most k

  // 3. collect every key >= tau from the winners' shares (chunks whose
  // largest value is below tau's are skipped on their packed value keys; at
  // about one chunk per thread a worklist, as in collect_tiles, measured
  // slower here)
  const uint32_t tv = (uint32_t)(tau >> 32);
  for (int64_t p0 = 0; p0 < (int64_t)W * R; p0 += kBatch * kThreads) {
    u32x4 v[kBatch];
    int64_t c[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t p = p0 + u * kThreads + t, pp = p < (int64_t)W * R ? p : 0;
      c[u] = S.winners[pp / R] + (pp % R) * kThreads;
      if (p >= (int64_t)W * R) c[u] = nchunks;
      v[u] = load16(rs, c[u] < nfull ? (uint32_t)(c[u] * 16) : kFar);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (c[u] >= nchunks) continue;
      uint64_t kk[8];
      if (c[u] < nfull) {
        if (chunk_value(v[u]) < tv) continue;
        full_keys(v[u], (uint32_t)(8 * c[u]), kk);
      } else {
        part_keys(rs, (uint32_t)(8 * c[u]), (uint32_t)n, kk);
      }
      uint32_t mask = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) mask |= (kk[e] >= tau && kk[e] != 0) ? 1u << e : 0u;
      if (mask) {
        const uint32_t at = atomicAdd(&S.count, (uint32_t)__builtin_popcount(mask));
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((mask >> e) & 1u) coll[at + __builtin_popcount(mask & ((1u << e) - 1u))] = kk[e];
      }
    }
  }
  __syncthreads();
}

// Steps 1-3 from the per-tile maximum keys that the greedy GEMV variant
// stored for the output projection's row tiles (tile i: rows row0(i) ..
// row0(i) + rows(i) - 1, large tiles of rpt rows first, then tiles of srows).
// The keys are exact and distinct, so tau = the k-th largest tile key (two
// value histograms, then the tied keys ranked), the k tiles with keys >= tau
// are the winners, and their rows are read in pieces of up to 8.  Returns
// false (for the whole workgroup) when the tied keys or the collected keys
// would not fit in `cap` entries of coll.
__device__ __forceinline__ bool collect_tiles(Lds& S, uint64_t* cands, uint64_t* coll, int cap, const uint16_t* logits, int64_t n,
                              const uint64_t* slots, int ntiles, int nbig, int rpt, int srows, int k) {
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  if (t < 256) S.hist1[t] = S.hist2[t] = 0u;
  if (t == 0) S.count = S.nwin = S.ntie = S.over = S.nwl = 0u;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(slots, (uint32_t)ntiles * 8u);  // past the end: key 0
  // Up to kBatch * kThreads tiles the keys stay in registers for every pass
  // below (one memory round trip); more are read again for each pass.
  const bool resident = ntiles <= kBatch * kThreads;
  uint64_t res[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u)
    res[u] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rk, (uint32_t)(u * kThreads + t) * 8u, 0, 0));
  auto keys = [&](int i0, uint64_t* v) {  // tile keys i0 + u * kThreads + t
    if (resident) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = res[u];
    } else {
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        v[u] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(
                                                rk, (uint32_t)(i0 + u * kThreads + t) * 8u, 0, 0));
    }
  };
  __syncthreads();

  uint64_t tau = 1;  // every real key is >= 1
  if (ntiles > k) {
    for (int i0 = 0; i0 < ntiles; i0 += kBatch * kThreads) {
      uint64_t v[kBatch];
      keys(i0, v);
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (v[u]) atomicAdd(&S.hist1[(uint32_t)(v[u] >> 40) & 0xFFu], 1u);
    }
    __syncthreads();
    if (wave == 0) suffix_select(S.hist1, (uint32_t)k, &S.bin1, &S.above1);
    __syncthreads();
    const uint32_t b1 = S.bin1;
    for (int i0 = 0; i0 < ntiles; i0 += kBatch * kThreads) {
      uint64_t v[kBatch];
      keys(i0, v);
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (v[u] && ((uint32_t)(v[u] >> 40) & 0xFFu) == b1) atomicAdd(&S.hist2[(uint32_t)(v[u] >> 32) & 0xFFu], 1u);
    }
    __syncthreads();
    if (wave == 0) suffix_select(S.hist2, (uint32_t)k - S.above1, &S.bin2, &S.above2);
    __syncthreads();
    const uint64_t v16 = ((uint64_t)b1 << 8) | S.bin2;
    const uint32_t m = (uint32_t)k - S.above1 - S.above2;  // tied keys to take (>= 1)
    const uint32_t ceq = S.hist2[S.bin2];
    if (ceq == m) {
      tau = v16 << 32;  // exactly the k largest tile keys have value >= v16
    } else {
      if (ceq > (uint32_t)cap) {  // uniform: ceq is the same for every thread
        __syncthreads();            // every thread has read the histograms before a fallback resets them
        return false;
      }
      for (int i0 = 0; i0 < ntiles; i0 += kBatch * kThreads) {
        uint64_t v[kBatch];
        keys(i0, v);
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          if (v[u] && (v[u] >> 32) == v16) coll[atomicAdd(&S.ntie, 1u)] = v[u];
      }
      __syncthreads();
      if (ceq <= (uint32_t)kRankMax) {
        if (t < (int)ceq) {
          const uint64_t key = coll[t];
          uint32_t rank = 0;
          for (uint32_t j = 0; j < ceq; ++j) rank += coll[j] > key;
          if (rank == m - 1) S.tau = key;
        }
      } else {
        int P = 1;
        while (P < (int)ceq) P <<= 1;
        for (int i = (int)ceq + t; i < P; i += kThreads) coll[i] = 0;
        __syncthreads();
        bitonic_desc(coll, P);
        if (t == 0) S.tau = coll[m - 1];
      }
      __syncthreads();
      tau = S.tau;
    }
  }
  for (int i0 = 0; i0 < ntiles; i0 += kBatch * kThreads) {
    uint64_t v[kBatch];
    keys(i0, v);
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (v[u] && v[u] >= tau) S.winners[atomicAdd(&S.nwin, 1u)] = i0 + u * kThreads + t;
  }
  __syncthreads();
  const int W = (int)S.nwin;  // k, or every tile when there are at most k

  // every key >= tau of the winners' rows; piece j of a winner = its rows
  // 8j .. 8j + 7 (one 16-byte load when they start on a multiple of 8).
  // Pieces whose largest value reaches tau's go to a worklist (in `cands`,
  // free until step 4), then one thread per listed piece forms its keys.
  const int maxp = (max(rpt, srows) + 7) / 8;
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(logits, (uint32_t)(n * 2));
  const uint32_t tv = (uint32_t)(tau >> 32);
  uint32_t* wl = reinterpret_cast<uint32_t*>(cands);
  auto piece = [&](int p, uint32_t& start, uint32_t& end) {  // rows of piece p (empty past the list)
    const int pp = p < W * maxp ? p : 0;
    const int i = S.winners[pp / maxp], j = pp % maxp;
    const int r0 = i < nbig ? i * rpt : nbig * rpt + (i - nbig) * srows;
    const int r1 = min(r0 + (i < nbig ? rpt : srows), (int)n);
    start = p < W * maxp ? (uint32_t)min(r0 + 8 * j, r1) : 0u;
    end = p < W * maxp ? (uint32_t)min(r0 + 8 * j + 8, r1) : 0u;
  };
  for (int p0 = 0; p0 < W * maxp; p0 += kBatch * kThreads) {
    u32x4 v[kBatch];
    uint32_t start[kBatch], end[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {  // branch-free: see step 1
      piece(p0 + u * kThreads + t, start[u], end[u]);
      const bool whole = end[u] == start[u] + 8 && (start[u] & 7u) == 0;
      v[u] = load16(ry, whole ? start[u] * 2u : kFar);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool whole = end[u] == start[u] + 8 && (start[u] & 7u) == 0;
      if (end[u] > start[u] && (!whole || chunk_value(v[u]) >= tv)) {
        const uint32_t at = atomicAdd(&S.nwl, 1u);
        if (at < (uint32_t)kWl) wl[at] = (uint32_t)(p0 + u * kThreads + t);
        else S.over = 1u;
      }
    }
  }
  __syncthreads();
  if (S.over) {        // uniform
    __syncthreads();   // every thread has read S.over before a fallback resets it
    return false;
  }
  const int nwl = (int)S.nwl;
  for (int w = t; w < nwl; w += kThreads) {
    uint32_t start, end;
    piece((int)wl[w], start, end);
    uint64_t kk[8];
    if (end == start + 8 && (start & 7u) == 0) full_keys(load16(ry, start * 2u), start, kk);
    else part_keys(ry, start, end, kk);
    uint32_t mask = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) mask |= (kk[e] >= tau && kk[e] != 0) ? 1u << e : 0u;
    if (mask) {
      const uint32_t at = atomicAdd(&S.count, (uint32_t)__builtin_popcount(mask));
      if (at + (uint32_t)__builtin_popcount(mask) > (uint32_t)cap) {
        S.over = 1u;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((mask >> e) & 1u) coll[at + __builtin_popcount(mask & ((1u << e) - 1u))] = kk[e];
      }
    }
  }
  __syncthreads();
  const bool ok = S.over == 0u;
  __syncthreads();  // every thread has read S.over before a fallback resets the state
  return ok;
}

// Steps 4-6 on coll[0, S.count): candidates, recomputed logits, token.
__device__ __forceinline__ void finish(Lds& S, uint64_t* cands, uint64_t* coll, const uint16_t* head, const uint16_t* x, int64_t K,
                       int k, int32_t* token, int32_t* cand, float* cand_logits) {
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  // 4. the k largest collected keys, in greedy order (keys are distinct)
  const int total = (int)S.count;
  if (total <= kRankMax) {
    if (t < total) {
      const uint64_t key = coll[t];
      int rank = 0;
      for (int j = 0; j < total; ++j) rank += coll[j] > key;
      if (rank < k) cands[rank] = key;
    }
  } else {
    int P = 1;
    while (P < total) P <<= 1;
    for (int i = total + t; i < P; i += kThreads) coll[i] = 0;
    __syncthreads();
    bitonic_desc(coll, P);
    for (int j = t; j < k; j += kThreads) cands[j] = coll[j];
  }
  __syncthreads();

  // 5. recompute the k candidates' logits: four rows per wave at a time, two
  // 16-byte chunks of each per lane in flight
  const int64_t kchunks = K / 8;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)(K * 2));
  for (int j0 = wave; j0 < k; j0 += 4 * (kThreads / 64)) {
    __amdgpu_buffer_rsrc_t rh[4];
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * (kThreads / 64);
      const uint32_t row = j < k ? key_row(cands[j]) : 0u;  // wave-uniform: one LDS word per wave
      rh[u] = make_rsrc_uniform(reinterpret_cast<const char*>(head + (int64_t)row * K), 0u,
                                j < k ? (uint32_t)(K * 2) : 0u);
    }
    for (int64_t q = lane; q < kchunks; q += 128) {
      // chunks q and q + 64; past the row's end the loads return zeros
      u32x4 xv[2], hv[4][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) xv[h] = load16(rx, (uint32_t)((q + 64 * h) * 16));
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h) hv[u][h] = load16(rh[u], (uint32_t)((q + 64 * h) * 16));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc[u] = fmaf(half_lo(hv[u][h][w]), half_lo(xv[h][w]), acc[u]);
            acc[u] = fmaf(half_hi(hv[u][h][w]), half_hi(xv[h][w]), acc[u]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float sum = wave_sum(acc[u]);
      const int j = j0 + u * (kThreads / 64);
      if (lane == 0 && j < k) S.exact[j] = sum;
    }
  }
  __syncthreads();

  // 6. the candidate with the largest recomputed logit
  uint64_t b = 0;
  for (int j = t; j < k; j += kThreads) {
    const uint32_t row = key_row(cands[j]);
    const uint64_t kk = key_f32(S.exact[j], row);
    b = kk > b ? kk : b;
    if (cand) cand[j] = (int32_t)row;
    if (cand_logits) cand_logits[j] = S.exact[j];
  }
  b = wave_max64(b);
  if (lane == 0) S.wave_best[wave] = b;
  __syncthreads();
  if (t == 0) {
    uint64_t m = S.wave_best[0];
    for (int w = 1; w < kThreads / 64; ++w) m = S.wave_best[w] > m ? S.wave_best[w] : m;
    *token = (int32_t)key_row(m);
  }
}

__global__ __launch_bounds__(kThreads) void head_rescore_kernel(const uint16_t* __restrict__ logits, int64_t n,
                                                                const uint16_t* __restrict__ head,
                                                                const uint16_t* __restrict__ x, int64_t K, int k,
                                                                int32_t* __restrict__ token, int32_t* __restrict__ cand,
                                                                float* __restrict__ cand_logits) {
  extern __shared__ uint64_t lds[];
  __shared__ Lds S;
  uint64_t* cands = lds;            // [kThreads]: the candidates, in greedy order
  uint64_t* coll = lds + kThreads;  // [collection capacity], power of two
  collect_shares(S, cands, coll, logits, n, k);
  finish(S, cands, coll, head, x, K, k, token, cand, cand_logits);
}

// After the greedy GEMV variant: the target's stored logits, x and tile
// geometry come from its descriptor, the per-tile keys from `slots`.  When
// the tile keys leave too many keys to collect (ties, large tiles), the
// selection starts again from the logits alone.
__global__ __launch_bounds__(kThreads) void gemv_rescore_kernel(const tkq_gemv_desc* __restrict__ descs, int count,
                                                                int target, int tiles,
                                                                const uint64_t* __restrict__ slots,
                                                                const uint16_t* __restrict__ head, int k,
                                                                int32_t* __restrict__ token, int32_t* __restrict__ cand,
                                                                float* __restrict__ cand_logits) {
  extern __shared__ uint64_t lds[];
  __shared__ Lds S;
  uint64_t* cands = lds;
  uint64_t* coll = lds + kThreads;  // TKQ_RESCORE_CAP entries
  const tkq_gemv_desc* d = descs + target;
  const int n = d->N;
  const int ntiles = (target + 1 < count ? descs[target + 1].work0 : tiles) - d->work0;
  const uint16_t* y = reinterpret_cast<const uint16_t*>(d->y);
  if (!collect_tiles(S, cands, coll, TKQ_RESCORE_CAP, y, n, slots, ntiles, d->big_tiles, d->rows_per_tile, d->small_rows,
                     k))
    collect_shares(S, cands, coll, y, n, k);
  finish(S, cands, coll, head, reinterpret_cast<const uint16_t*>(d->x), d->K, k, token, cand, cand_logits);
}

}  // namespace

// Raises a kernel's dynamic-LDS limit above the 64 KB default, once per
// kernel (which = 0, 1) and device: the attribute is set on the current
// device, so each device the library runs on needs its own call.
static hipError_t allow_lds(const void* fn, int which, int bytes) {
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> raised[2][kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && raised[which][dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && dev >= 0 && dev < kMaxDevices) raised[which][dev].store(true, std::memory_order_release);
  return e;
}

int64_t rescore_capacity(int64_t n, int k) {
  const int64_t R = ((n + 7) / 8 + kThreads - 1) / kThreads;
  return (int64_t)k * R * 8;
}

hipError_t launch_head_rescore(const uint16_t* logits, int64_t n, const uint16_t* head, const uint16_t* x,
                               int64_t K, int k, int32_t* token, int32_t* cand, float* cand_logits,
                               hipStream_t stream) {
  int64_t P = 1;
  while (P < rescore_capacity(n, k)) P <<= 1;
  const size_t lds = (size_t)(kThreads + P) * 8;
  if (lds > 64 * 1024) {  // above the default dynamic-LDS limit
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(head_rescore_kernel), 0,
                                   (kThreads + TKQ_RESCORE_CAP) * 8);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(head_rescore_kernel, dim3(1), dim3(kThreads), lds, stream, logits, n, head, x, K, k, token,
                     cand, cand_logits);
  return hipGetLastError();
}

hipError_t launch_gemv_rescore(const tkq_gemv_desc* dev_descs, int count, int target, int64_t tiles,
                               const uint64_t* slots, const uint16_t* head, int k, int32_t* token, int32_t* cand,
                               float* cand_logits, hipStream_t stream) {
  const size_t lds = (size_t)(kThreads + TKQ_RESCORE_CAP) * 8;
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(gemv_rescore_kernel), 1, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemv_rescore_kernel, dim3(1), dim3(kThreads), lds, stream, dev_descs, count, target, (int)tiles,
                     slots, head, k, token, cand, cand_logits);
  return hipGetLastError();
}

}  // namespace tkq

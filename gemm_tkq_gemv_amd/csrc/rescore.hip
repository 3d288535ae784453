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
#include "device_common.h"
#include "kernels.h"

namespace tkq {

namespace {

constexpr int kThreads = 1024;
constexpr int kInFlight = 16;    // 16-byte loads a thread issues before using any
constexpr int kRankMax = 256;    // collections up to this size are ranked by counting

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

// Keys of the 8 logits of chunk c (logits 8c .. 8c+7); 0 for those at or
// past n.  A full chunk is one 16-byte load, the ragged last one 2-byte loads.
__device__ __forceinline__ void chunk_keys(__amdgpu_buffer_rsrc_t rs, int64_t c, int64_t n, int64_t nfull,
                                           uint64_t kk[8]) {
  if (c < nfull) {
    const u32x4 v = load16(rs, (uint32_t)(c * 16));
#pragma unroll
    for (int e = 0; e < 8; ++e) kk[e] = key_f16((e & 1) ? (v[e >> 1] >> 16) : v[e >> 1], (uint32_t)(8 * c + e));
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t i = 8 * c + e;
      kk[e] = i < n ? key_f16(load2(rs, (uint32_t)(i * 2)), (uint32_t)i) : 0;
    }
  }
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

// Wave 0: the largest bin b of hist[256] whose suffix count S(b) (bins >= b)
// reaches `need`, and S(b + 1); need >= 1 and S(0) >= need.
__device__ __forceinline__ void suffix_select(const uint32_t* hist, uint32_t need, uint32_t* bin,
                                              uint32_t* above) {
  const int lane = threadIdx.x & 63;
  uint32_t h[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = hist[4 * lane + i];
    sum += h[i];
  }
  uint32_t s = sum;  // -> sum over lanes >= lane
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_down(s, o, 64);
    if (lane + o < 64) s += u;
  }
  int mine = -1;
  uint32_t suf = s;  // S(4 lane + i) as i goes up
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (suf >= need) mine = 4 * lane + i;
    suf -= h[i];
  }
  int b = mine;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) b = max(b, __shfl_xor(b, o, 64));
  if (lane == (b >> 2)) {
    uint32_t sb = s;
    for (int i = 0; i < (b & 3); ++i) sb -= h[i];
    *bin = (uint32_t)b;
    *above = sb - h[b & 3];
  }
}

__global__ __launch_bounds__(kThreads) void head_rescore_kernel(const uint16_t* __restrict__ logits, int64_t n,
                                                                const uint16_t* __restrict__ head,
                                                                const uint16_t* __restrict__ x, int64_t K, int k,
                                                                int32_t* __restrict__ token, int32_t* __restrict__ cand,
                                                                float* __restrict__ cand_logits) {
  extern __shared__ uint64_t lds[];
  uint64_t* cands = lds;             // [kThreads]: the candidates, in greedy order
  uint64_t* coll = lds + kThreads;   // [collection capacity], power of two
  __shared__ uint32_t hist1[256], hist2[256];
  __shared__ uint32_t count, nwin, ntie, bin1, above1, bin2, above2;  // counters zeroed below
  __shared__ unsigned long long tau_s;
  __shared__ int32_t winners[kThreads];
  __shared__ float exact[TKQ_RESCORE_MAX_K];
  __shared__ unsigned long long wave_best[kThreads / 64];

  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int64_t nchunks = (n + 7) / 8, nfull = n / 8;
  const int64_t R = (nchunks + kThreads - 1) / kThreads;  // chunks per share
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(logits, (uint32_t)(n * 2));
  if (t < 256) hist1[t] = hist2[t] = 0u;
  if (t == 0) count = nwin = ntie = 0u;

  // 1. this thread's share maximum value.  Every round but the last holds a
  // full chunk for every thread; the last one may hold a full, a ragged or no
  // chunk.
  u16x2 vmax = {0, 0}, vmin = {0xFFFF, 0xFFFF};
  const int64_t Rfull = R - 1;
  for (int64_t r0 = 0; r0 < Rfull; r0 += kInFlight) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      if (r0 + u < Rfull) v[u] = load16(rs, (uint32_t)((t + (r0 + u) * kThreads) * 16));
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
  if (M) atomicAdd(&hist1[M >> 8], 1u);
  __syncthreads();
  if (wave == 0) {
    uint32_t nonempty = 0;
    for (int i = lane; i < 256; i += 64) nonempty += hist1[i];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) nonempty += __shfl_xor(nonempty, o, 64);
    if (nonempty <= (uint32_t)k) {  // at most k non-empty shares: take them all
      if (lane == 0) bin1 = 0xFFFFFFFFu;
    } else {
      suffix_select(hist1, (uint32_t)k, &bin1, &above1);
    }
  }
  __syncthreads();
  uint64_t tau = 1;  // every real key is >= 1
  bool winner = M != 0;
  if (bin1 != 0xFFFFFFFFu) {
    if (M && (M >> 8) == bin1) atomicAdd(&hist2[M & 0xFFu], 1u);
    __syncthreads();
    if (wave == 0) suffix_select(hist2, (uint32_t)k - above1, &bin2, &above2);
    __syncthreads();
    const uint32_t v16 = (bin1 << 8) | bin2;
    const uint32_t m = (uint32_t)k - above1 - above2;  // shares of maximum v16 to take (>= 1)
    winner = M > v16;
    if (hist2[bin2] == m) {
      // exactly m shares have maximum v16: all of them are winners, and the
      // keys of value >= v16 lie in the k winners' shares only
      tau = (uint64_t)v16 << 32;
      winner = M >= v16;
    } else {
      // more: each tied share's first row of value v16 decides.  The tied
      // shares (listed in `winners`) are read again, their first keys of
      // value v16 max-reduced into `cands`; both are free until later steps.
      uint32_t my = 0;
      if (M == v16) {
        my = atomicAdd(&ntie, 1u);
        winners[my] = t;
        cands[my] = 0;
      }
      __syncthreads();
      const int nt = (int)ntie;
      for (int64_t p = t; p < (int64_t)nt * R; p += kThreads) {
        const int64_t c = winners[p / R] + (p % R) * kThreads;
        if (c >= nchunks) continue;
        uint64_t kk[8];
        chunk_keys(rs, c, n, nfull, kk);
        uint64_t f = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) f = (kk[e] >> 32) == v16 && kk[e] > f ? kk[e] : f;
        if (f) atomicMax(reinterpret_cast<unsigned long long*>(&cands[p / R]), (unsigned long long)f);
      }
      __syncthreads();
      if (M == v16) {
        const uint64_t mine = cands[my];
        uint32_t rank = 0;
        for (int j = 0; j < nt; ++j) rank += cands[j] > mine;
        if (rank == m - 1) tau_s = mine;
        winner = rank < m;
      }
      __syncthreads();
      tau = tau_s;
    }
  }
  if (winner) winners[atomicAdd(&nwin, 1u)] = t;
  __syncthreads();
  const int W = (int)nwin;  // k, or every non-empty share when there are at most k

  // 3. collect every key >= tau from the winners' shares
  for (int64_t p = t; p < (int64_t)W * R; p += kThreads) {
    const int64_t c = winners[p / R] + (p % R) * kThreads;
    if (c >= nchunks) continue;
    uint64_t kk[8];
    chunk_keys(rs, c, n, nfull, kk);
    uint32_t mask = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) mask |= (kk[e] >= tau && kk[e] != 0) ? 1u << e : 0u;
    if (mask) {
      const uint32_t at = atomicAdd(&count, (uint32_t)__builtin_popcount(mask));
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((mask >> e) & 1u) coll[at + __builtin_popcount(mask & ((1u << e) - 1u))] = kk[e];
    }
  }
  __syncthreads();

  // 4. the k largest collected keys, in greedy order (keys are distinct)
  const int total = (int)count;
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
      float sum = acc[u];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
      const int j = j0 + u * (kThreads / 64);
      if (lane == 0 && j < k) exact[j] = sum;
    }
  }
  __syncthreads();

  // 6. the candidate with the largest recomputed logit
  uint64_t b = 0;
  for (int j = t; j < k; j += kThreads) {
    const uint32_t row = key_row(cands[j]);
    const uint64_t kk = key_f32(exact[j], row);
    b = kk > b ? kk : b;
    if (cand) cand[j] = (int32_t)row;
    if (cand_logits) cand_logits[j] = exact[j];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t hi = __shfl_xor((uint32_t)(b >> 32), o, 64);
    const uint32_t lo = __shfl_xor((uint32_t)b, o, 64);
    const uint64_t other = ((uint64_t)hi << 32) | lo;
    b = other > b ? other : b;
  }
  if (lane == 0) wave_best[wave] = b;
  __syncthreads();
  if (t == 0) {
    uint64_t m = wave_best[0];
    for (int w = 1; w < kThreads / 64; ++w) m = wave_best[w] > m ? wave_best[w] : m;
    *token = (int32_t)key_row(m);
  }
}

}  // namespace

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
  if (lds > 64 * 1024) {  // above the default dynamic-LDS limit (once; idempotent)
    static bool raised = false;
    if (!raised) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(head_rescore_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (kThreads + TKQ_RESCORE_CAP) * 8);
      if (e != hipSuccess) return e;
      raised = true;
    }
  }
  hipLaunchKernelGGL(head_rescore_kernel, dim3(1), dim3(kThreads), lds, stream, logits, n, head, x, K, k, token,
                     cand, cand_logits);
  return hipGetLastError();
}

}  // namespace tkq

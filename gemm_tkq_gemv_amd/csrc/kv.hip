// Low-bit KV cache and single-query decode attention for gfx950 (the
// BitDecoding README: 4-bit KV codes in groups of 128, K quantized per channel
// and V per token, head dimension 128; one decode step attends one query over
// a long cache, which makes it another HBM-bound stream like the weight GEMV).
//
// Storage (one (batch, KV head) = a sequence of 128-token pages):
//   K codes  uint32 [128 tokens][16]   4-bit, channel c of token t at
//                                      word 16t + c/8, bits 4(c%8)
//   V codes  uint32 [128 channels][16] 4-bit, token t of channel c at
//                                      word 2048 + 16c + t/8, bits 4(t%8)
//   K meta   uint32 [128]              half2 {scale, zero} per channel
//   V meta   uint32 [128]              half2 {scale, zero} per token
// V is channel-major so that the value product, like the scores, reads whole
// rows front to back with 16-byte loads.
//
// Decode (one workgroup = a split of the pages of one KV head for up to four
// query heads; wave w takes pages w, w + 4, ...):
//  * Scores are a GEMV over the page's tokens: with per-channel scales,
//    s_t = sum_c q_c sK_c (k_tc - zK_c) = sum_c q'_c k_tc - sum_c q'_c zK_c,
//    q' = q * sK rounded to fp16 once per page; 4 lanes per token (32
//    channels each), 16 tokens per wave step, the int4 magic-number unpack
//    and v_dot2_f32_f16.
//  * Online softmax over pages in fp32 (exp2 of log2-scaled scores).
//  * The value product is a GEMV over the page's channels: with per-token
//    scales, o_c = sum_t p_t sV_t (v_ct - zV_t) = sum_t p'_t v_ct - sum_t
//    p'_t zV_t, p' = p * sV rounded to fp16 (in LDS, read back in the unpack
//    order); 4 lanes per channel (32 tokens each).
//  * Exact unpack: a code field OR-ed into fp16 1024.0 (low nibble, ulp 1)
//    or 64.0 (high nibble, ulp 1/16) gives M + code; subtracting M + zero in
//    fp16 leaves code - zero exactly, so every product is a small exact
//    integer times q' or p' and the fp32 sums carry only the dequantized
//    terms (removing M * sum x after the sum instead left an error that grows
//    with M |x|: a query channel of ~1e3 on zero-point keys broke the
//    tolerance).
//  * Each workgroup writes (m, l, o[128]) per query head to a workspace.
//    With few splits (short contexts) it counts its arrival and the last
//    split of each (sequence, head group) to arrive merges the splits
//    (log-sum-exp) and stores fp16, so a decode step is one launch; with
//    more, a second kernel merges them.
//  * Per-sequence lengths: pages past a sequence's length are skipped and
//    the tokens past it in its last page get score -inf.
#include "device_common.h"
#include "kernels.h"

namespace tkq {

namespace {

constexpr int kD = 128, kPage = 128;
constexpr int kPageWords = 4352;  // (8192 + 8192 + 512 + 512) / 4
constexpr int kKC = 0, kVC = 2048, kKM = 4096, kVM = 4224;
constexpr int kWaves = 4;
constexpr uint32_t kMagic = 0x64006400u;
constexpr float kLog2e = 1.4426950408889634f;

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

// ------------------------------------------------------------------ pack --
// Same arithmetic as the int4 g128 weight packer: lo = min(min, 0),
// hi = max(max, 0), s = fp16((hi - lo) / 15) (0 -> 1), z = clamp(rint(-lo / s),
// 0, 15), q = clamp(rint(x / s) + z, 0, 15).
__device__ __forceinline__ uint32_t quant_group(const float* v, int stride, uint8_t* q, int qstride) {
  float lo = 0.0f, hi = 0.0f;
  for (int i = 0; i < 128; ++i) {
    lo = fminf(lo, v[i * stride]);
    hi = fmaxf(hi, v[i * stride]);
  }
  _Float16 h = (_Float16)((hi - lo) / 15.0f);
  if (h == (_Float16)0.0f) h = (_Float16)1.0f;
  const float s = (float)h;
  const float z = fminf(fmaxf(rintf(-lo / s), 0.0f), 15.0f);
  for (int i = 0; i < 128; ++i) q[i * qstride] = (uint8_t)(int)fminf(fmaxf(rintf(v[i * stride] / s) + z, 0.0f), 15.0f);
  return (uint32_t)__builtin_bit_cast(uint16_t, h) | ((uint32_t)half_bits(z) << 16);
}

// Valid tokens of sequence b: lens[b] clamped to [0, T] (all T without lens).
__device__ __forceinline__ int seq_len(const int32_t* lens, int b, int T) {
  return lens ? min(max(lens[b], 0), T) : T;
}

// One workgroup (256 threads) per page; K and V are fp16 [B][T][Hk][128].
// Tokens at or past the sequence's length are quantized as zeros: K groups
// (a channel over the page) already span 0, so their scale and zero-point
// are those of the valid tokens alone; such a V token is an all-zero group.
__global__ __launch_bounds__(256) void kv_pack_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                      const int32_t* __restrict__ lens, int T, int Hk,
                                                      uint32_t* __restrict__ cache) {
  __shared__ float tile[kPage * (kD + 1)];
  __shared__ uint8_t codes[kPage * kD];
  const int p = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int P = T / kPage;
  uint32_t* page = cache + (((size_t)b * Hk + hk) * P + p) * kPageWords;
  const int valid = seq_len(lens, b, T) - kPage * p;  // valid tokens of this page (may be <= 0 or > 128)
  for (int part = 0; part < 2; ++part) {
    const uint16_t* src = part == 0 ? K : V;
    // tile[t][c] = value of token 128p + t, channel c
    for (int i = threadIdx.x; i < kPage * kD; i += 256) {
      const int t = i / kD, c = i - t * kD;
      const uint16_t bits = t < valid ? src[(((size_t)b * T + (size_t)kPage * p + t) * Hk + hk) * kD + c] : 0;
      tile[t * (kD + 1) + c] = (float)__builtin_bit_cast(_Float16, bits);
    }
    __syncthreads();
    if (threadIdx.x < 128) {
      const int g = threadIdx.x;
      if (part == 0)  // K: group = channel g over the tokens; codes[t][c]
        page[kKM + g] = quant_group(tile + g, kD + 1, codes + g, kD);
      else            // V: group = token g over the channels; codes[t][c]
        page[kVM + g] = quant_group(tile + g * (kD + 1), 1, codes + g * kD, 1);
    }
    __syncthreads();
    for (int w = threadIdx.x; w < 2048; w += 256) {
      uint32_t word = 0;
      if (part == 0) {  // token-major: word 16t + j holds channels 8j..8j+7 of token t
        const int t = w >> 4, j = w & 15;
        for (int i = 0; i < 8; ++i) word |= (uint32_t)codes[t * kD + 8 * j + i] << (4 * i);
        page[kKC + w] = word;
      } else {          // channel-major: word 16c + j holds tokens 8j..8j+7 of channel c
        const int c = w >> 4, j = w & 15;
        for (int i = 0; i < 8; ++i) word |= (uint32_t)codes[(8 * j + i) * kD + c] << (4 * i);
        page[kVC + w] = word;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- decode --
struct Regs {
  uint32_t m0, m1, magic, magic64;
};
constexpr uint32_t kMagic64 = 0x54005400u;  // fp16 pair (64.0, 64.0)

// sum over one 16-byte chunk (32 codes, natural nibble order) of
// (code - zero) * x with the GEMV's pairing (0,4),(1,5),(2,6),(3,7):
// zs[4w + i] = (M + z, M + z') for the chunk positions (8w + i, 8w + i + 4),
// M = 1024 for the low nibble fields (i even) and 64 for the high ones.
__device__ __forceinline__ float chunk_dot(u32x4 q, const uint32_t* xr, const uint32_t* zs, const Regs& R) {
  float acc = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t v = q[w], t = v >> 8;
    acc = __builtin_amdgcn_fdot2(as_h2((v & R.m0) | R.magic) - as_h2(zs[4 * w + 0]), as_h2(xr[4 * w + 0]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2((v & R.m1) | R.magic64) - as_h2(zs[4 * w + 1]), as_h2(xr[4 * w + 1]), acc,
                                 false);
    acc = __builtin_amdgcn_fdot2(as_h2((t & R.m0) | R.magic) - as_h2(zs[4 * w + 2]), as_h2(xr[4 * w + 2]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2((t & R.m1) | R.magic64) - as_h2(zs[4 * w + 3]), as_h2(xr[4 * w + 3]), acc,
                                 false);
  }
  return acc;
}

// The subtrahends of chunk_dot for the 32 chunk positions whose zero points
// are the high halves of meta[0..31] (half2 {scale, zero} words); with
// `mixed` the high nibble positions take 64 (chunk_dot), else all take 1024
// (the matrix-core kernel's multiplier-1 unpack).
__device__ __forceinline__ void chunk_zeros(const uint32_t* meta, bool mixed, const Regs& R, uint32_t* zs) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t zz = __builtin_amdgcn_perm(meta[8 * w + i + 4], meta[8 * w + i], 0x07060302u);
      const uint32_t mg = (mixed && (i & 1)) ? R.magic64 : R.magic;
      zs[4 * w + i] = __builtin_bit_cast(uint32_t, as_h2(zz) + as_h2(mg));
    }
  }
}

// 32 natural-order fp16 values (16 words, 2 per word) -> the pairing order.
__device__ __forceinline__ void pair_order(const uint32_t* raw, uint32_t* xr) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t a = raw[4 * w], b = raw[4 * w + 1], c = raw[4 * w + 2], d = raw[4 * w + 3];
    xr[4 * w + 0] = __builtin_amdgcn_perm(c, a, 0x05040100u);  // (x0, x4)
    xr[4 * w + 1] = __builtin_amdgcn_perm(c, a, 0x07060302u);  // (x1, x5)
    xr[4 * w + 2] = __builtin_amdgcn_perm(d, b, 0x05040100u);  // (x2, x6)
    xr[4 * w + 3] = __builtin_amdgcn_perm(d, b, 0x07060302u);  // (x3, x7)
  }
}

// Cross-lane steps without the LDS pipe: DPP within rows of 16 lanes, and
// gfx950's permlane swaps across rows (with the value in both operands, the
// two results hold each lane's own value and that of lane ^ 16 or ^ 32).
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(u32(v), u32(v), false, false);
  return fmaxf(f32(r[0]), f32(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(u32(v), u32(v), false, false);
  return fmaxf(f32(r[0]), f32(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(u32(v), u32(v), false, false);
  return f32(r[0]) + f32(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(u32(v), u32(v), false, false);
  return f32(r[0]) + f32(r[1]);
}
__device__ __forceinline__ float quad_sum(float v) {  // lanes ^ 1, then ^ 2: the total in all four
  v += dppf<kQuadSwap1>(v);
  v += dppf<kQuadSwap2>(v);
  return v;
}
// The matrix-core kernel's waves raise their priority while they issue a
// page's loads, so that they are not queued behind other waves' unpack and
// MFMA work (32/8 heads: +3 % at 32k and 128k tokens; the vector-ALU kernel
// measured 1 % slower with it and does not).
__device__ __forceinline__ void prio_on() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void prio_off() { __builtin_amdgcn_s_setprio(0); }
// Whole-wave max / sum in every lane: quads, then the mirrors within 8 and
// 16 lanes (the halves being uniform by then), then across rows.
__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dppf<kQuadSwap1>(v));
  v = fmaxf(v, dppf<kQuadSwap2>(v));
  v = fmaxf(v, dppf<kRowHalfMirror>(v));
  v = fmaxf(v, dppf<kRowMirror>(v));
  return max_xor32(max_xor16(v));
}
__device__ __forceinline__ float wave_sum_f(float v) {
  v += dppf<kQuadSwap1>(v);
  v += dppf<kQuadSwap2>(v);
  v += dppf<kRowHalfMirror>(v);
  v += dppf<kRowMirror>(v);
  return sum_xor32(sum_xor16(v));
}

// Partial results cross workgroups on different XCDs, whose L2 caches are
// not coherent with each other: they are written and read with device-scope
// (sc1) accesses, which go to the device-coherent level, so no cache
// write-back or invalidation (a release/acquire fence) is needed.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Splits up to which the decode merges its partials in the kernel itself
// (the last split of a head group to finish does it); with more, one more
// launch (kv_merge_kernel) spreads the merge over every (sequence, head).
constexpr int kFuseMaxSplits = 16;

// The arrival of one split of a (sequence, head group): its partial
// (o[128], m, l per head) is in ws.  Every wave waits until its partial
// stores are performed, then one thread counts the workgroup's arrival; the
// last of the `splits` (<= kFuseMaxSplits) workgroups to arrive merges the
// partials (log-sum-exp; a thread's loads are all issued before any is
// used), stores fp16 out and resets the counter to 0 for the next call.  No
// workgroup waits for another.
__device__ __forceinline__ void arrive_and_merge(const float* ws, uint32_t* counter, int splits, int bh0, int ng,
                                                 uint16_t* __restrict__ out) {
  __shared__ int is_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    is_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (uint32_t)(splits - 1);
  __syncthreads();
  if (!is_last) return;
  for (int i = threadIdx.x; i < ng * kD; i += 256) {
    const int g = i / kD, c = i - g * kD;
    const float* w = ws + (size_t)(bh0 + g) * splits * (kD + 2);
    float ms[kFuseMaxSplits], ls[kFuseMaxSplits], os[kFuseMaxSplits];
#pragma unroll
    for (int sp = 0; sp < kFuseMaxSplits; ++sp) {
      const float* ws_sp = w + (size_t)(sp < splits ? sp : 0) * (kD + 2);  // always in range
      ms[sp] = ld_dev(ws_sp + kD);
      ls[sp] = ld_dev(ws_sp + kD + 1);
      os[sp] = ld_dev(ws_sp + c);
    }
    float M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < kFuseMaxSplits; ++sp)
      if (sp < splits) M = fmaxf(M, ms[sp]);
    float O = 0.0f, L = 0.0f;
#pragma unroll
    for (int sp = 0; sp < kFuseMaxSplits; ++sp) {
      const float a = sp >= splits || ms[sp] == -INFINITY ? 0.0f : exp2f(ms[sp] - M);
      L = fmaf(ls[sp], a, L);
      O = fmaf(os[sp], a, O);
    }
    out[(size_t)(bh0 + g) * kD + c] = half_bits(L > 0.0f ? O / L : 0.0f);  // no valid token: 0
  }
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct WaveLds {
  uint32_t meta[256];           // K meta [128 channels] then V meta [128 tokens]
  uint32_t qv[kKvMaxGroup][kD / 2];  // query heads, fp16 pairs in natural order
  uint32_t pv[1][kPage / 2];    // p' of the current head, fp16 pairs in natural order
  float o[kKvMaxGroup][kD];     // unnormalised outputs per head (in LDS: registers stay
                                // independent of the number of heads)
};

// KUP (one query head only): the page's K codes are requested in the same
// round trip as its metadata.  The registers they take cost a wave per SIMD
// (134 VGPRs): measured +7 % when every wave has one page, -11 % with two,
// so the host picks it by pages per wave.
template <int G, bool KUP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G == 1 && !KUP ? 4 : 1, 8))) void kv_decode_kernel(
    const uint16_t* __restrict__ q,
                                                        const uint32_t* __restrict__ cache,
                                                        const int32_t* __restrict__ lens, int H, int Hk, int P,
                                                        int pages_per_split, float scale_log2,
                                                        float* __restrict__ ws, int splits,
                                                        uint32_t* __restrict__ counters, uint16_t* __restrict__ out) {
  __shared__ WaveLds lds[kWaves];
  __shared__ float merge[kWaves][G][kD + 2];
  constexpr bool kKUp = KUP && G == 1;
  const int split = blockIdx.x, hsub = blockIdx.y, b = blockIdx.z;
  const int gq = H / Hk;                        // query heads per KV head
  const int hk = (hsub * G) / gq;               // this workgroup's KV head
  const int h0 = hsub * G;                      // first query head
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int quad = lane >> 2, sub = lane & 3;
  WaveLds& L = lds[wave];
  const Regs R = {in_sgpr(0x000F000Fu), in_sgpr(0x00F000F0u), in_vgpr(kMagic), in_vgpr(kMagic64)};

  // query heads -> LDS (fp16 pairs)
  for (int i = lane; i < G * kD / 2; i += 64) {
    const int g = i / (kD / 2), w = i - g * (kD / 2);
    L.qv[g][w] = reinterpret_cast<const uint32_t*>(q + ((size_t)b * H + h0 + g) * kD)[w];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

  float m[G], l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
  }
  for (int i = lane; i < G * kD; i += 64) L.o[i / kD][i % kD] = 0.0f;

  const int len = seq_len(lens, b, P * kPage);
  const int p0 = split * pages_per_split, p1 = min((len + kPage - 1) / kPage, p0 + pages_per_split);
  const uint32_t* base = cache + ((size_t)b * Hk + hk) * (size_t)P * kPageWords;
  for (int p = p0 + wave; p < p1; p += kWaves) {
    const __amdgpu_buffer_rsrc_t pg = make_rsrc(base + (size_t)p * kPageWords, kPageWords * 4u);
    const int valid = len - kPage * p;  // tokens t >= valid are past the sequence (last page only)
    // page metadata -> LDS (one 16-byte load per lane covers all 256 words)
    const u32x4 mt = load16(pg, (uint32_t)(kKM + 4 * lane) * 4u);
    u32x4 kall[kKUp ? 8 : 1];
    if constexpr (kKUp) {
#pragma unroll
      for (int i = 0; i < 8; ++i) kall[i] = load16_nt(pg, (uint32_t)(kKC + 16 * (16 * i + quad) + 4 * sub) * 4u);
    }
    *reinterpret_cast<u32x4*>(&L.meta[4 * lane]) = mt;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // The query heads one after another: the page comes from HBM for the
    // first and from the caches for the others.
#pragma unroll
    for (int g = 0; g < G; ++g) {
      // ---- scores: lane chunk = channels 32 sub .. 32 sub + 31 of token 16 st + quad
      float sc[8];
      {
        uint32_t qp[16];
        {
          uint32_t raw[16], sp[16], qr[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {  // (s_2i, s_2i+1) of the chunk's channels, and the query
            raw[i] = __builtin_amdgcn_perm(L.meta[32 * sub + 2 * i + 1], L.meta[32 * sub + 2 * i], 0x05040100u);
            qr[i] = L.qv[g][16 * sub + i];
          }
          pair_order(raw, sp);
          pair_order(qr, qp);
#pragma unroll
          for (int i = 0; i < 16; ++i) qp[i] = __builtin_bit_cast(uint32_t, as_h2(qp[i]) * as_h2(sp[i]));
        }
        uint32_t zk[16];  // M + zK of the chunk's channels
        chunk_zeros(&L.meta[32 * sub], true, R, zk);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 kc[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (kKUp) kc[i] = kall[kKUp ? 4 * half + i : 0];
            else kc[i] = load16_nt(pg, (uint32_t)(kKC + 16 * (16 * (4 * half + i) + quad) + 4 * sub) * 4u);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = quad_sum(chunk_dot(kc[i], qp, zk, R)) * scale_log2;
            sc[4 * half + i] = 16 * (4 * half + i) + quad < valid ? v : -INFINITY;
          }
        }
      }

      // ---- online softmax (base 2), p' = p * sV to LDS
      float valpha;
      {
        float pm = sc[0];
#pragma unroll
        for (int st = 1; st < 8; ++st) pm = fmaxf(pm, sc[st]);
        pm = wave_max_f(pm);
        const float mn = fmaxf(m[g], pm);
        const float alpha = exp2f(m[g] - mn);  // 0 on the first page (m = -inf)
        m[g] = mn;
        float ps = 0.0f;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const int t = 16 * st + quad;
          const float pt = exp2f(sc[st] - mn);
          const uint32_t vm = L.meta[128 + t];
          const _Float16 pp = (_Float16)(pt * half_lo(vm));  // p' = p * sV
          if (sub == 0) {
            ps += pt;
            reinterpret_cast<_Float16*>(L.pv[0])[t] = pp;
          }
        }
        l[g] = l[g] * alpha + wave_sum_f(ps);
        valpha = alpha;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

      // ---- value product: lane chunk = tokens 32 sub .. 32 sub + 31 of channel 16 st + quad
      {
        uint32_t zv[16];  // M + zV of the chunk's tokens
        chunk_zeros(&L.meta[128 + 32 * sub], true, R, zv);
        uint32_t pp[16];
        {
          uint32_t praw[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) praw[i] = L.pv[0][16 * sub + i];
          pair_order(praw, pp);
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 vc[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vc[i] = load16_nt(pg, (uint32_t)(kVC + 16 * (16 * (4 * half + i) + quad) + 4 * sub) * 4u);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float d = quad_sum(chunk_dot(vc[i], pp, zv, R));
            if (sub == 0) {
              float& oc = L.o[g][16 * (4 * half + i) + quad];
              oc = fmaf(oc, valpha, d);
            }
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_sched_barrier(0);  // heads one after another: no overlap of their working sets
    }
  }

  // ---- merge the four waves, then write this split's partial result
  for (int i = lane; i < G * kD; i += 64) merge[wave][i / kD][i % kD] = L.o[i / kD][i % kD];
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      merge[wave][g][kD] = m[g];
      merge[wave][g][kD + 1] = l[g];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * kD; i += 256) {
    const int g = i / kD, c = i - g * kD;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, merge[w][g][kD]);
    float Lsum = 0.0f, O = 0.0f;
    for (int w = 0; w < kWaves; ++w) {
      const float a = merge[w][g][kD] == -INFINITY ? 0.0f : exp2f(merge[w][g][kD] - M);
      Lsum += merge[w][g][kD + 1] * a;
      O += merge[w][g][c] * a;
    }
    float* dst = ws + (((size_t)b * H + h0 + g) * splits + split) * (kD + 2);
    st_dev(dst + c, O);
    if (c == 0) {
      st_dev(dst + kD, M);
      st_dev(dst + kD + 1, Lsum);
    }
  }
  if (counters) arrive_and_merge(ws, counters + (size_t)b * gridDim.y + hsub, splits, b * H + h0, G, out);
}

// ------------------------------------------------- decode, grouped queries --
// With several query heads per KV head the two products are small GEMMs
// (16 tokens x 128 channels x up to 16 heads per MFMA block), so they run on
// the matrix cores and the work per page no longer grows with the group:
//  * scores: A = K codes (lane l: token l % 16 of a 16-token block, channels
//    32 (l / 16) .. +31 = one 16-byte chunk), unpacked with multiplier 1 only
//    (four shifts per word) into (1024 + k) fp16 pairs minus (1024 + zK)
//    (exact: k - zK); B = q' = q * sK (lane l: head l % 16, the same 32
//    channels), in the unpack's k order.  D[token][head] is the score.
//  * softmax per head in the lanes of that head's column (l % 16), online
//    over pages; p' = p * sV goes through LDS, head-major.
//  * value product: A = V codes (lane l: channel l % 16 of a 16-channel
//    block, tokens 32 (l / 16) .. +31, minus 1024 + zV), B = p' (lane l:
//    head l % 16); D[channel][head] is the page's output, and each lane
//    keeps its head's 32 output values in registers.
//  * the four waves' partials (m, l, o) are combined in LDS and the
//    workgroup writes one partial per head and split; the last to arrive merges.
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One code word (8 nibbles, natural order) -> (c - z) fp16 values in the
// order (0, 4, 1, 5, 2, 6, 3, 7): OR into 1024.0, minus zs[i] = (1024 + z,
// 1024 + z') of the pair (i, i + 4), both exact.
__device__ __forceinline__ half8 unpack_exact(uint32_t w, uint32_t m, uint32_t magic, const uint32_t* zs) {
  h2 v[4] = {as_h2((w & m) | magic) - as_h2(zs[0]), as_h2(((w >> 4) & m) | magic) - as_h2(zs[1]),
             as_h2(((w >> 8) & m) | magic) - as_h2(zs[2]), as_h2(((w >> 12) & m) | magic) - as_h2(zs[3])};
  return __builtin_bit_cast(half8, v);
}
__device__ __forceinline__ half8 as_half8(const uint32_t* p) {
  u32x4 v = {p[0], p[1], p[2], p[3]};
  return __builtin_bit_cast(half8, v);
}


// LDS of the matrix-core kernel: the page loop's buffers, reused after it
// for the combination of the four waves' partials.
struct MfmaLoop {
  uint32_t qv[16][kD / 2];                               // query heads, fp16 pairs (zero past NG)
  uint32_t metas[kWaves][256];                           // K meta then V meta of the wave's page
  __attribute__((aligned(16))) _Float16 pvs[kWaves][16][kPage];  // p' per head
};
union MfmaLds {
  MfmaLoop loop;
  float part[kWaves][16][kD + 2];  // per wave and head: o[128], m, l
};

// NG: query heads of this workgroup (1..16, padded to 16 MFMA columns).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void kv_decode_mfma_kernel(
    const uint16_t* __restrict__ q, const uint32_t* __restrict__ cache, const int32_t* __restrict__ lens, int H,
    int Hk, int P, int pages_per_split, float scale_log2, float* __restrict__ ws, int splits, int NG,
    uint32_t* __restrict__ counters, uint16_t* __restrict__ out) {
  __shared__ MfmaLds lds;
  auto& qv = lds.loop.qv;
  const int split = blockIdx.x, hsub = blockIdx.y, b = blockIdx.z;
  const int gq = H / Hk;
  const int h0 = hsub * NG, hk = h0 / gq;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 15, blk = lane >> 4;
  const uint32_t M4 = in_sgpr(0x000F000Fu), magic = in_vgpr(kMagic);
  const Regs R = {M4, M4, magic, magic};  // chunk_zeros with multiplier 1 only
  for (int i = threadIdx.x; i < 16 * (kD / 2); i += 256) {
    const int g = i / (kD / 2), w = i - g * (kD / 2);
    qv[g][w] = g < NG ? reinterpret_cast<const uint32_t*>(q + ((size_t)b * H + h0 + g) * kD)[w] : 0u;
  }
  __syncthreads();
  uint32_t* meta = lds.loop.metas[wave];
  _Float16* pv = lds.loop.pvs[wave][col];

  float m = -INFINITY, l = 0.0f;  // this lane's head (col)
  f32x4 o[8];                      // channels 16 cb + 4 blk + r of head col
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

  const int len = seq_len(lens, b, P * kPage);
  const int p0 = split * pages_per_split, p1 = min((len + kPage - 1) / kPage, p0 + pages_per_split);
  const uint32_t* base = cache + ((size_t)b * Hk + hk) * (size_t)P * kPageWords;
  for (int p = p0 + wave; p < p1; p += kWaves) {
    const __amdgpu_buffer_rsrc_t pg = make_rsrc(base + (size_t)p * kPageWords, kPageWords * 4u);
    const int valid = len - kPage * p;  // tokens t >= valid are past the sequence (last page only)
    // the K codes are requested before the metadata is stored to LDS, so
    // both arrive in one round trip
    prio_on();
    const u32x4 mt = load16(pg, (uint32_t)(kKM + 4 * lane) * 4u);
    u32x4 kc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kc[i] = load16_nt(pg, (uint32_t)(kKC + 16 * (16 * i + col) + 4 * blk) * 4u);
    prio_off();
    *reinterpret_cast<u32x4*>(&meta[4 * lane]) = mt;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    // ---- q' = q * sK for head col, channels 32 blk .. +31, and 1024 + zK of those channels
    uint32_t qb[16], zk[16];
    chunk_zeros(&meta[32 * blk], false, R, zk);
    {
      uint32_t sraw[16], qraw[16], sp[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sraw[i] = __builtin_amdgcn_perm(meta[32 * blk + 2 * i + 1], meta[32 * blk + 2 * i], 0x05040100u);
        qraw[i] = qv[col][16 * blk + i];
      }
      pair_order(sraw, sp);
      pair_order(qraw, qb);
#pragma unroll
      for (int i = 0; i < 16; ++i) qb[i] = __builtin_bit_cast(uint32_t, as_h2(qb[i]) * as_h2(sp[i]));
    }

    // ---- scores: 8 blocks of 16 tokens; lane holds tokens 16 tb + 4 blk + r of head col
    float sc[8][4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half == 1) {
        prio_on();
#pragma unroll
        for (int i = 0; i < 4; ++i) kc[i] = load16_nt(pg, (uint32_t)(kKC + 16 * (16 * (4 + i) + col) + 4 * blk) * 4u);
        prio_off();
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
        const u32x4 kw = kc[i];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(unpack_exact(kw[j], M4, magic, zk + 4 * j), as_half8(qb + 4 * j),
                                                     d, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sc[4 * half + i][r] = 16 * (4 * half + i) + 4 * blk + r < valid ? d[r] * scale_log2 : -INFINITY;
      }
    }
    // the first half of the V codes is requested before the softmax
    u32x4 vc[4];
    prio_on();
#pragma unroll
    for (int i = 0; i < 4; ++i) vc[i] = load16_nt(pg, (uint32_t)(kVC + 16 * (16 * i + col) + 4 * blk) * 4u);
    prio_off();

    // ---- online softmax for head col
    float pm = sc[0][0];
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) pm = fmaxf(pm, sc[tb][r]);
    }
    pm = max_xor32(max_xor16(pm));
    const float mn = fmaxf(m, pm);
    const float alpha = exp2f(m - mn);  // 0 on the first page (m = -inf)
    m = mn;
    float ps = 0.0f;
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tb + 4 * blk + r;
        const float pt = exp2f(sc[tb][r] - mn);
        const uint32_t vm = meta[128 + t];
        const _Float16 pp = (_Float16)(pt * half_lo(vm));  // p' = p * sV
        pv[t] = pp;
        ps += pt;
      }
    }
    ps = sum_xor32(sum_xor16(ps));
    l = l * alpha + ps;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    // ---- value product: B = p' of head col, tokens 32 blk .. +31 (A minus 1024 + zV of those tokens)
    uint32_t pb[16], zv[16];
    chunk_zeros(&meta[128 + 32 * blk], false, R, zv);
    {
      uint32_t praw[16];
      const uint32_t* src = reinterpret_cast<const uint32_t*>(pv) + 16 * blk;
#pragma unroll
      for (int i = 0; i < 16; ++i) praw[i] = src[i];
      pair_order(praw, pb);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half == 1) {
        prio_on();
#pragma unroll
        for (int i = 0; i < 4; ++i) vc[i] = load16_nt(pg, (uint32_t)(kVC + 16 * (16 * (4 + i) + col) + 4 * blk) * 4u);
        prio_off();
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
        const u32x4 vw = vc[i];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(unpack_exact(vw[j], M4, magic, zv + 4 * j), as_half8(pb + 4 * j),
                                                     d, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) o[4 * half + i][r] = fmaf(o[4 * half + i][r], alpha, d[r]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }

  // ---- combine the four waves' partials, then write this split's partial per head
  __syncthreads();  // every wave is done with the loop's LDS
  if (col < NG) {
    float* pw = lds.part[wave][col];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) pw[16 * cb + 4 * blk + r] = o[cb][r];
    }
    if (blk == 0) {
      pw[kD] = m;
      pw[kD + 1] = l;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NG * kD; i += 256) {
    const int g = i / kD, c = i - g * kD;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds.part[w][g][kD]);
    float Lsum = 0.0f, O = 0.0f;
    for (int w = 0; w < kWaves; ++w) {
      const float a = lds.part[w][g][kD] == -INFINITY ? 0.0f : exp2f(lds.part[w][g][kD] - M);
      Lsum += lds.part[w][g][kD + 1] * a;
      O += lds.part[w][g][c] * a;
    }
    float* dst = ws + (((size_t)b * H + h0 + g) * splits + split) * (kD + 2);
    st_dev(dst + c, O);
    if (c == 0) {
      st_dev(dst + kD, M);
      st_dev(dst + kD + 1, Lsum);
    }
  }
  if (counters) arrive_and_merge(ws, counters + (size_t)b * gridDim.y + hsub, splits, b * H + h0, NG, out);
}

// One workgroup per (b, head): merge the splits, normalise, store fp16
// (decodes with more than kFuseMaxSplits splits).
// 512 threads = 4 groups of 128 channels; the splits are taken 512 at a time
// (weights exp2(m_s - M) in LDS) and dealt round-robin to the groups, whose
// sums meet in LDS at the end.  Maxima and sums over threads: within each
// wave by shuffles, then over the 8 waves in LDS.
constexpr int kMergeThreads = 512, kMergeGroups = kMergeThreads / kD, kMergeWaves = kMergeThreads / 64;
__global__ __launch_bounds__(kMergeThreads) void kv_merge_kernel(const float* __restrict__ ws, int splits,
                                                                 uint16_t* __restrict__ out) {
  __shared__ float wgt[kMergeThreads];
  __shared__ float osum[kMergeGroups][kD];
  __shared__ float wmax[kMergeWaves], wsum[kMergeWaves];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int c = tid % kD, grp = tid / kD, wv = tid >> 6;
  const float* w = ws + (size_t)bh * splits * (kD + 2);
  float mloc = -INFINITY;
  for (int s = tid; s < splits; s += kMergeThreads) mloc = fmaxf(mloc, w[s * (kD + 2) + kD]);
  mloc = wave_max_f(mloc);
  if ((tid & 63) == 0) wmax[wv] = mloc;
  __syncthreads();
  float M = wmax[0];
#pragma unroll
  for (int i = 1; i < kMergeWaves; ++i) M = fmaxf(M, wmax[i]);
  float O = 0.0f, lloc = 0.0f;
  for (int base = 0; base < splits; base += kMergeThreads) {
    const int s = base + tid;
    float a = 0.0f;
    if (s < splits) {
      const float ms = w[s * (kD + 2) + kD];
      a = ms == -INFINITY ? 0.0f : exp2f(ms - M);
      lloc += w[s * (kD + 2) + kD + 1] * a;
    }
    if (base > 0) __syncthreads();  // the previous chunk's weights are consumed
    wgt[tid] = a;
    __syncthreads();
    const int n = min(kMergeThreads, splits - base);
    const float* col = w + (size_t)base * (kD + 2) + c;
#pragma unroll 8
    for (int i = grp; i < n; i += kMergeGroups) O = fmaf(wgt[i], col[(size_t)i * (kD + 2)], O);
  }
  osum[grp][c] = O;
  lloc = wave_sum_f(lloc);
  if ((tid & 63) == 0) wsum[wv] = lloc;
  __syncthreads();
  if (grp == 0) {
    float L = 0.0f, t = 0.0f;
#pragma unroll
    for (int i = 0; i < kMergeWaves; ++i) L += wsum[i];
#pragma unroll
    for (int j = 0; j < kMergeGroups; ++j) t += osum[j][c];
    out[(size_t)bh * kD + c] = half_bits(L > 0.0f ? t / L : 0.0f);  // no valid token: 0
  }
}

}  // namespace

hipError_t launch_kv_pack(const uint16_t* K, const uint16_t* V, const int32_t* lens, int B, int T, int Hk,
                          uint32_t* cache, hipStream_t stream) {
  hipLaunchKernelGGL(kv_pack_kernel, dim3((uint32_t)(T / kPage), (uint32_t)Hk, (uint32_t)B), dim3(256), 0, stream, K,
                     V, lens, T, Hk, cache);
  return hipGetLastError();
}

// Grouped queries (at least 3 query heads per KV head) take the matrix-core
// kernel.
bool kv_use_mfma(int H, int Hk) { return H / Hk >= 3; }

// Query heads per workgroup: the whole group if it fits (8 heads for the
// vector-ALU kernel, 16 for the matrix-core one), else its largest divisor
// that does.
int kv_heads_per_wg(int H, int Hk) {
  const int G = H / Hk;
  const int cap = kv_use_mfma(H, Hk) ? 16 : kKvMaxGroup;
  for (int gb = G < cap ? G : cap; gb > 1; --gb)
    if (G % gb == 0) return gb;
  return 1;
}

int kv_splits(int B, int H, int Hk, int T, int cus, int* pages_per_split) {
  const int P = T / kPage;
  const int gb = kv_heads_per_wg(H, Hk);
  const int64_t groups = (int64_t)B * (H / gb);
  // enough workgroups for about 4 per CU (every wave streams its own pages;
  // the merge of more splits costs little), at least one page per wave
  const int per_cu = 4;
  int64_t want = ((int64_t)per_cu * cus + groups - 1) / groups;
  int64_t max_splits = (P + kWaves - 1) / kWaves;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  const int pps = (int)((P + want - 1) / want);
  *pages_per_split = pps;
  return (P + pps - 1) / pps;
}

hipError_t launch_kv_decode(const uint16_t* q, const uint32_t* cache, const int32_t* lens, int B, int H, int Hk,
                            int T, float sm_scale, uint16_t* out, float* ws, uint32_t* counters, int splits,
                            int pages_per_split, hipStream_t stream) {
  const int P = T / kPage;
  const int gb = kv_heads_per_wg(H, Hk);
  const dim3 grid((uint32_t)splits, (uint32_t)(H / gb), (uint32_t)B);
  const float sl2 = sm_scale * kLog2e;
  uint32_t* cnt = splits <= kFuseMaxSplits ? counters : nullptr;  // fused merge, else a merge launch
  if (kv_use_mfma(H, Hk)) {
    hipLaunchKernelGGL(kv_decode_mfma_kernel, grid, dim3(256), 0, stream, q, cache, lens, H, Hk, P, pages_per_split,
                       sl2, ws, splits, gb, cnt, out);
  } else {
    switch (gb) {
#define TKQ_KV_CASE(G)                                                                                           \
  case G:                                                                                                       \
    hipLaunchKernelGGL(kv_decode_kernel<G>, grid, dim3(256), 0, stream, q, cache, lens, H, Hk, P, pages_per_split, \
                       sl2, ws, splits, cnt, out);                                                              \
    break;
      case 1:
        if (pages_per_split <= kWaves)  // one page per wave: K codes with the metadata
          hipLaunchKernelGGL((kv_decode_kernel<1, true>), grid, dim3(256), 0, stream, q, cache, lens, H, Hk, P,
                             pages_per_split, sl2, ws, splits, cnt, out);
        else
          hipLaunchKernelGGL((kv_decode_kernel<1, false>), grid, dim3(256), 0, stream, q, cache, lens, H, Hk, P,
                             pages_per_split, sl2, ws, splits, cnt, out);
        break;
      TKQ_KV_CASE(2)
      TKQ_KV_CASE(3)
      TKQ_KV_CASE(4)
      TKQ_KV_CASE(5)
      TKQ_KV_CASE(6)
      TKQ_KV_CASE(7)
      TKQ_KV_CASE(8)
#undef TKQ_KV_CASE
      default:
        return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || cnt) return e;
  hipLaunchKernelGGL(kv_merge_kernel, dim3((uint32_t)(B * H)), dim3(kMergeThreads), 0, stream, ws, splits, out);
  return hipGetLastError();
}

}  // namespace tkq

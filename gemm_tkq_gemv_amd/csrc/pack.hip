// Quantize-and-pack kernels for gfx950.
//
// One wavefront handles one 128-weight group of one row: each lane reads two
// adjacent fp32 weights (a coalesced 512-byte read per wave), the group
// statistics are reduced across the wave, and every lane writes its own
// codes.  All arithmetic is IEEE fp32 with true division, rint (round half to
// even) and round-to-nearest-even fp16 conversion, so the codes and metadata
// are bit-identical to a plain fp32 evaluation of the same steps.
//
// Quantizers (the pages print no formulas; these are the readings of the
// Whetstone README, "What the weights can actually survive" for int4 g128 and
// ternary g128, and of TKintegers K5, "What is K5?" for the K5 byte code):
//   int4 g128 : lo = min(min w, 0), hi = max(max w, 0), s = fp16((hi-lo)/15),
//               z = clamp(rint(-lo/s), 0, 15), q = clamp(rint(w/s) + z, 0, 15)
//   K5        : s = fp16(max|w| / 121), c = clamp(rint(w/s), -121, 121) + 121
//   ternary   : s = fp16(sequential-sum|w| / 128), code = clamp(rint(w/s),-1,1)+1
//   int2 g128 : as int4 with 4 levels: s = fp16((hi-lo)/3), z, q in 0..3
//   int3 g128 : as int4 with 8 levels: s = fp16((hi-lo)/7), z, q in 0..7,
//               stored plane-major for the GEMV's loads (see tkq.h)
//   int4 hier-g32 (Whetstone README, quantizer table "group 32 with
//               hierarchical scale metadata"; "Prior art", the Q4_K
//               comparison): per 32-group s_g = (hi-lo)/15, m_g = -lo; per
//               row d = fp16(max s_g / 15), dmin = fp16(max m_g / 15);
//               sc = clamp(rint(s_g/d), 1, 15), mi = clamp(rint(m_g/dmin), 0, 15),
//               q = clamp(rint((w + dmin*mi) / (d*sc)), 0, 15)
// A scale that rounds to fp16 zero is stored as 1.0 (Whetstone README, status
// list: the underflowing fp16 row scale).
#include "device_common.h"
#include "kernels.h"

namespace tkq {

namespace {

constexpr int kGroup = 128;
constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ float guard_scale(float s, uint16_t* bits) {
  _Float16 h = (_Float16)s;
  if (h == (_Float16)0.0f) h = (_Float16)1.0f;
  *bits = __builtin_bit_cast(uint16_t, h);
  return (float)h;
}

__device__ __forceinline__ bool group_of_wave(int64_t groups, int64_t* g) {
  *g = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  return *g < groups;
}

__global__ __launch_bounds__(256) void pack_int4_kernel(const float* __restrict__ W, int64_t K,
                                                        int64_t groups, uint8_t* __restrict__ codes,
                                                        uint32_t* __restrict__ meta) {
  int64_t g;
  if (!group_of_wave(groups, &g)) return;
  const int lane = threadIdx.x & 63;
  const int64_t gpr = K / kGroup;
  const int64_t row = g / gpr, col = (g - row * gpr) * kGroup;
  const float2 w = *reinterpret_cast<const float2*>(W + row * K + col + 2 * lane);
  const float lo = fminf(wave_min(fminf(w.x, w.y)), 0.0f);
  const float hi = fmaxf(wave_max(fmaxf(w.x, w.y)), 0.0f);
  uint16_t sbits;
  const float s = guard_scale((hi - lo) / 15.0f, &sbits);
  const int z = (int)fminf(fmaxf(rintf(-lo / s), 0.0f), 15.0f);
  const float zf = (float)z;
  const int q0 = (int)fminf(fmaxf(rintf(w.x / s) + zf, 0.0f), 15.0f);
  const int q1 = (int)fminf(fmaxf(rintf(w.y / s) + zf, 0.0f), 15.0f);
  // elements 2*lane, 2*lane+1 are nibbles (2*lane)%8, +1 of word (2*lane)/8:
  // little-endian, so byte `lane` of the row's group block.
  codes[row * (K / 2) + col / 2 + lane] = (uint8_t)(q0 | (q1 << 4));
  if (lane == 0) meta[g] = (uint32_t)sbits | ((uint32_t)half_bits(zf) << 16);
}

__global__ __launch_bounds__(256) void pack_int2_kernel(const float* __restrict__ W, int64_t K,
                                                        int64_t groups, uint8_t* __restrict__ codes,
                                                        uint32_t* __restrict__ meta) {
  int64_t g;
  if (!group_of_wave(groups, &g)) return;
  const int lane = threadIdx.x & 63;
  const int64_t gpr = K / kGroup;
  const int64_t row = g / gpr, col = (g - row * gpr) * kGroup;
  const float2 w = *reinterpret_cast<const float2*>(W + row * K + col + 2 * lane);
  const float lo = fminf(wave_min(fminf(w.x, w.y)), 0.0f);
  const float hi = fmaxf(wave_max(fmaxf(w.x, w.y)), 0.0f);
  uint16_t sbits;
  const float s = guard_scale((hi - lo) / 3.0f, &sbits);
  const float zf = (float)(int)fminf(fmaxf(rintf(-lo / s), 0.0f), 3.0f);
  const int q0 = (int)fminf(fmaxf(rintf(w.x / s) + zf, 0.0f), 3.0f);
  const int q1 = (int)fminf(fmaxf(rintf(w.y / s) + zf, 0.0f), 3.0f);
  // 2-bit fields: elements 2*lane, 2*lane+1 form nibble `lane` of the group's
  // 32 bytes; lanes 2m and 2m+1 share byte m.
  const int nib = q0 | (q1 << 2);
  const int other = __shfl_xor(nib, 1, 64);
  if ((lane & 1) == 0) codes[row * (K / 4) + col / 4 + (lane >> 1)] = (uint8_t)(nib | (other << 4));
  if (lane == 0) meta[g] = (uint32_t)sbits | ((uint32_t)half_bits(zf) << 16);
}

// int3: the wave's 128 codes go through LDS; lanes 0..11 each build one of
// the group's 12 words and store it into its plane.
__global__ __launch_bounds__(256) void pack_int3_kernel(const float* __restrict__ W, int64_t K, int64_t groups,
                                                        uint32_t* __restrict__ codes, uint32_t* __restrict__ meta) {
  __shared__ uint8_t cs[kWavesPerBlock][kGroup];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  int64_t g;
  const bool live = group_of_wave(groups, &g);
  const int64_t gpr = K / kGroup;
  const int64_t row = live ? g / gpr : 0, grp = live ? g - row * gpr : 0;
  float2 w = make_float2(0.0f, 0.0f);
  if (live) w = *reinterpret_cast<const float2*>(W + row * K + grp * kGroup + 2 * lane);
  const float lo = fminf(wave_min(fminf(w.x, w.y)), 0.0f);
  const float hi = fmaxf(wave_max(fmaxf(w.x, w.y)), 0.0f);
  uint16_t sbits;
  const float s = guard_scale((hi - lo) / 7.0f, &sbits);
  const float zf = (float)(int)fminf(fmaxf(rintf(-lo / s), 0.0f), 7.0f);
  cs[wave][2 * lane] = (uint8_t)(int)fminf(fmaxf(rintf(w.x / s) + zf, 0.0f), 7.0f);
  cs[wave][2 * lane + 1] = (uint8_t)(int)fminf(fmaxf(rintf(w.y / s) + zf, 0.0f), 7.0f);
  __syncthreads();
  if (!live) return;
  if (lane < 12) {
    const int b = lane / 3, j = lane - 3 * b;
    const uint8_t* c = cs[wave] + 32 * b;
    uint32_t word = 0;
#pragma unroll
    for (int f = 0; f < 5; ++f) word |= ((uint32_t)c[10 * j + f] << (3 * f)) | ((uint32_t)c[10 * j + 5 + f] << (16 + 3 * f));
    word |= ((uint32_t)(c[30] >> j) & 1u) << 15;
    word |= ((uint32_t)(c[31] >> j) & 1u) << 31;
    // plane lane / 4 (planes of N rows of K/8 bytes), word lane % 4 of this
    // group's 16 bytes in that plane's row
    const int64_t row_words = K / 32, rows = groups / gpr;
    codes[((lane >> 2) * rows + row) * row_words + 4 * grp + (lane & 3)] = word;
  }
  if (lane == 0) meta[g] = (uint32_t)sbits | ((uint32_t)half_bits(zf) << 16);
}

__global__ __launch_bounds__(256) void pack_k5_kernel(const float* __restrict__ W, int64_t K,
                                                      int64_t groups, uint8_t* __restrict__ codes,
                                                      uint16_t* __restrict__ scale) {
  int64_t g;
  if (!group_of_wave(groups, &g)) return;
  const int lane = threadIdx.x & 63;
  const int64_t gpr = K / kGroup;
  const int64_t row = g / gpr, col = (g - row * gpr) * kGroup;
  const float2 w = *reinterpret_cast<const float2*>(W + row * K + col + 2 * lane);
  const float a = wave_max(fmaxf(fabsf(w.x), fabsf(w.y)));
  uint16_t sbits;
  const float s = guard_scale(a / 121.0f, &sbits);
  const int c0 = (int)fminf(fmaxf(rintf(w.x / s), -121.0f), 121.0f) + 121;
  const int c1 = (int)fminf(fmaxf(rintf(w.y / s), -121.0f), 121.0f) + 121;
  *reinterpret_cast<uint16_t*>(codes + row * K + col + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) scale[g] = sbits;
}

__global__ __launch_bounds__(256) void pack_tern_kernel(const float* __restrict__ W, int64_t K,
                                                        int64_t groups, uint8_t* __restrict__ codes,
                                                        uint16_t* __restrict__ scale) {
  __shared__ float absw[kWavesPerBlock][kGroup];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  int64_t g;
  const bool live = group_of_wave(groups, &g);
  float2 w = make_float2(0.0f, 0.0f);
  int64_t row = 0, col = 0;
  if (live) {
    const int64_t gpr = K / kGroup;
    row = g / gpr;
    col = (g - row * gpr) * kGroup;
    w = *reinterpret_cast<const float2*>(W + row * K + col + 2 * lane);
  }
  absw[wave][2 * lane] = fabsf(w.x);
  absw[wave][2 * lane + 1] = fabsf(w.y);
  __syncthreads();
  if (!live) return;
  // absmean with the sum taken strictly in k order (every lane reads the same
  // LDS words, so all lanes hold the identical total).
  float total = 0.0f;
#pragma unroll 8
  for (int k = 0; k < kGroup; ++k) total += absw[wave][k];
  uint16_t sbits;
  const float s = guard_scale(total / 128.0f, &sbits);
  const int t0 = (int)fminf(fmaxf(rintf(w.x / s), -1.0f), 1.0f) + 1;
  const int t1 = (int)fminf(fmaxf(rintf(w.y / s), -1.0f), 1.0f) + 1;
  // 2-bit fields: elements 2*lane, 2*lane+1 form nibble `lane` of the group's
  // 32 bytes; lanes 2m and 2m+1 share byte m.
  const int nib = t0 | (t1 << 2);
  const int other = __shfl_xor(nib, 1, 64);
  if ((lane & 1) == 0) codes[row * (K / 4) + col / 4 + (lane >> 1)] = (uint8_t)(nib | (other << 4));
  if (lane == 0) scale[g] = sbits;
}

// Minimum / maximum over each 32-lane half of the wave (one 32-weight group).
__device__ __forceinline__ float half_wave_min(float v) {
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) v = fminf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float half_wave_max(float v) {
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// int4 hier-g32: one wavefront per row (the row pair depends on every group
// of the row).  Each iteration covers 64 consecutive weights = two groups,
// one per half-wave; lane l reads weight 64i + l (coalesced).  Pass 1 finds
// the row maxima of the wanted step and offset, pass 2 re-reads the row and
// writes codes and indices.  Lanes past K (when K % 64 == 32) see w = 0,
// which contributes s = m = 0 to the maxima and writes nothing.
__global__ __launch_bounds__(256) void pack_hier_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ meta, int64_t rbase) {
  const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= N) return;
  const int lane = threadIdx.x & 63;
  const float* w = W + row * K;
  float smax = 0.0f, mmax = 0.0f;
  for (int64_t base = 0; base < K; base += 64) {
    const int64_t k = base + lane;
    const float v = k < K ? w[k] : 0.0f;
    const float lo = fminf(half_wave_min(v), 0.0f), hi = fmaxf(half_wave_max(v), 0.0f);
    smax = fmaxf(smax, (hi - lo) / 15.0f);
    mmax = fmaxf(mmax, -lo);
  }
  uint16_t dbits, mbits;
  const float d = guard_scale(wave_max(smax) / 15.0f, &dbits);
  const float dmin = guard_scale(wave_max(mmax) / 15.0f, &mbits);
  const int64_t ng = K / 32;
  for (int64_t base = 0; base < K; base += 64) {
    const int64_t k = base + lane;
    const bool ok = k < K;
    const float v = ok ? w[k] : 0.0f;
    const float lo = fminf(half_wave_min(v), 0.0f), hi = fmaxf(half_wave_max(v), 0.0f);
    const float sc = fminf(fmaxf(rintf(((hi - lo) / 15.0f) / d), 1.0f), 15.0f);
    const float mi = fminf(fmaxf(rintf(-lo / dmin), 0.0f), 15.0f);
    const float step = d * sc, off = dmin * mi;  // both exact
    const int q = (int)fminf(fmaxf(rintf((v + off) / step), 0.0f), 15.0f);
    const int other = __shfl_xor(q, 1, 64);
    if (ok && (lane & 1) == 0) codes[row * (K / 2) + (k >> 1)] = (uint8_t)(q | (other << 4));
    if (ok && (lane & 31) == 0) meta[row * ng + (k >> 5)] = (uint8_t)((int)sc | ((int)mi << 4));
  }
  if (lane == 0) *reinterpret_cast<uint32_t*>(meta + rbase + row * 4) = (uint32_t)dbits | ((uint32_t)mbits << 16);
  // zero padding between the group bytes and the row pairs
  if (row == 0 && N * ng + lane < rbase) meta[N * ng + lane] = 0;
}

// One thread per output word: 32 consecutive weights -> 32 sign bits.
__global__ __launch_bounds__(256) void pack_bin_kernel(const float* __restrict__ W, int64_t words,
                                                       uint32_t* __restrict__ bits) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= words) return;
  const float4* src = reinterpret_cast<const float4*>(W + t * 32);
  uint32_t b = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = src[i];
    b |= (uint32_t)(v.x < 0.0f) << (4 * i + 0);
    b |= (uint32_t)(v.y < 0.0f) << (4 * i + 1);
    b |= (uint32_t)(v.z < 0.0f) << (4 * i + 2);
    b |= (uint32_t)(v.w < 0.0f) << (4 * i + 3);
  }
  bits[t] = b;
}

}  // namespace

hipError_t launch_pack(int fmt, const float* W, int64_t N, int64_t K, void* codes, void* meta,
                       hipStream_t stream) {
  if (fmt == kFmtBin) {
    const int64_t words = N * (K / 32);
    const int64_t blocks = (words + 255) / 256;
    hipLaunchKernelGGL(pack_bin_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, W, words,
                       (uint32_t*)codes);
    return hipGetLastError();
  }
  if (fmt == kFmtHier) {
    const int64_t blocks = (N + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(pack_hier_kernel, dim3((uint32_t)blocks), dim3(64 * kWavesPerBlock), 0, stream, W, N, K,
                       (uint8_t*)codes, (uint8_t*)meta, hier_row_offset(N, K));
    return hipGetLastError();
  }
  const int64_t groups = N * (K / kGroup);
  const int64_t blocks = (groups + kWavesPerBlock - 1) / kWavesPerBlock;
  const dim3 grid((uint32_t)blocks), block(64 * kWavesPerBlock);
  switch (fmt) {
    case kFmtInt4:
      hipLaunchKernelGGL(pack_int4_kernel, grid, block, 0, stream, W, K, groups, (uint8_t*)codes,
                         (uint32_t*)meta);
      break;
    case kFmtInt3:
      hipLaunchKernelGGL(pack_int3_kernel, grid, block, 0, stream, W, K, groups, (uint32_t*)codes,
                         (uint32_t*)meta);
      break;
    case kFmtInt2:
      hipLaunchKernelGGL(pack_int2_kernel, grid, block, 0, stream, W, K, groups, (uint8_t*)codes,
                         (uint32_t*)meta);
      break;
    case kFmtK5:
      hipLaunchKernelGGL(pack_k5_kernel, grid, block, 0, stream, W, K, groups, (uint8_t*)codes,
                         (uint16_t*)meta);
      break;
    case kFmtTern:
      hipLaunchKernelGGL(pack_tern_kernel, grid, block, 0, stream, W, K, groups, (uint8_t*)codes,
                         (uint16_t*)meta);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tkq

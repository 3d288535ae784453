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
  const int64_t groups = N * (K / kGroup);
  const int64_t blocks = (groups + kWavesPerBlock - 1) / kWavesPerBlock;
  const dim3 grid((uint32_t)blocks), block(64 * kWavesPerBlock);
  switch (fmt) {
    case kFmtInt4:
      hipLaunchKernelGGL(pack_int4_kernel, grid, block, 0, stream, W, K, groups, (uint8_t*)codes,
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

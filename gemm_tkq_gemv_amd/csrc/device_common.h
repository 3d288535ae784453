// Device helpers shared by the gfx950 kernels of libtkq: buffer resources,
// 16-byte non-temporal loads, fp16 bit casts and DPP group reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tkq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Word 3 of a raw (untyped) buffer resource on gfx9-family parts: 32-bit
// data format, no swizzle, no stride.
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy bits of gfx950 buffer instructions: bit1 = non-temporal.
constexpr int kAuxNT = 2;

// A buffer resource covering [base, base + bytes).  Loads at offsets at or
// beyond `bytes` return zero and stores there are dropped, so out-of-range
// rows and chunks need no branches.  `base` and `bytes` must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// make_rsrc for [base + off, base + total) (empty past the end) from values
// the caller knows to be wave-uniform but the compiler may not: they are
// moved to scalar registers explicitly, so a load through the resource needs
// no per-lane loop over distinct descriptors.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const char* base, uint32_t off,
                                                                    uint32_t total) {
  const uint64_t p = reinterpret_cast<uint64_t>(base) + off;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(total > off ? total - off : 0u);
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), n);
}

__device__ __forceinline__ u32x4 load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxNT);
}
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ void store2(__amdgpu_buffer_rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ float f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t u32(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float half_lo(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
}
__device__ __forceinline__ uint16_t half_bits(float f) {  // fp32 -> fp16, nearest even
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// DPP controls (gfx9 encoding).
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kRowMirror = 0x140;     // lane i <- lane 15-i within 16
constexpr int kRowBcast15 = 0x142;    // row r <- lane 15 of row r-1
constexpr int kRowBcast31 = 0x143;    // row 3 (and 2) <- lane 31

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Sum over aligned groups of L lanes (L = 1 << lg, wave-uniform).  The group
// total is exact for integers; for floats the order is a fixed butterfly.
// The total is valid in the LAST lane of every group (lane % L == L - 1).
__device__ __forceinline__ float group_sum(float v, int lg) {
  if (lg >= 1) v += f32((uint32_t)dpp<kQuadSwap1>((int)u32(v)));
  if (lg >= 2) v += f32((uint32_t)dpp<kQuadSwap2>((int)u32(v)));
  if (lg >= 3) v += f32((uint32_t)dpp<kRowHalfMirror>((int)u32(v)));
  if (lg >= 4) v += f32((uint32_t)dpp<kRowMirror>((int)u32(v)));
  if (lg >= 5) v += f32((uint32_t)dpp<kRowBcast15, 0xA>((int)u32(v)));
  if (lg >= 6) v += f32((uint32_t)dpp<kRowBcast31, 0x8>((int)u32(v)));
  return v;
}
__device__ __forceinline__ int group_sum(int v, int lg) {
  if (lg >= 1) v += dpp<kQuadSwap1>(v);
  if (lg >= 2) v += dpp<kQuadSwap2>(v);
  if (lg >= 3) v += dpp<kRowHalfMirror>(v);
  if (lg >= 4) v += dpp<kRowMirror>(v);
  if (lg >= 5) v += dpp<kRowBcast15, 0xA>(v);
  if (lg >= 6) v += dpp<kRowBcast31, 0x8>(v);
  return v;
}

// Whole-wave min / max / sum with the result in every lane (butterfly over
// xor shuffles; order-independent for min and max).
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace tkq

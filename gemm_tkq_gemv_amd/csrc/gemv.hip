// Grouped low-bit GEMV for gfx950: y_i = dequant(W_i) . x_i for many
// independent matrices in one launch.
//
// Decode at batch 1 reads every weight once for one multiply-add, so the
// product is bound by HBM bandwidth (Whetstone README, "The one fact that
// shapes everything": tok/s ceiling = bandwidth / bytes per token).  The
// kernel is therefore organised around the byte stream:
//
//  * Work unit.  One workgroup (4 wave64s) owns a tile of consecutive rows of
//    one matrix (int4 g128 has its own kernel, gemv_int4_kernel, that reads
//    128-byte lines per 8-lane unit and keeps x in LDS); the grid is the
//    concatenation of every matrix's tiles, and a workgroup finds its matrix
//    by binary search over the descriptors' first-tile indices (scalar
//    loads).  Tiles are large (~24 KB per wave,
//    amortising the per-tile setup) except over the last stretch of the
//    sweep, where small tiles let the final workgroups finish together
//    instead of trailing one large tile's duration behind each other.
//  * Lanes.  L = 2^lg lanes share a row; lane `sub` of the group reads the
//    row's 16-byte chunks sub, sub+L, ... (J "passes"), so every load
//    instruction of the wave reads whole rows front to back: contiguous,
//    coalesced, non-temporal 128-bit buffer loads.  With S k-slices, S waves
//    split one row's chunks and combine through LDS.
//  * x stays in registers.  Each lane owns fixed chunk positions, so it loads
//    its slice of x once per tile and keeps it, pre-permuted to the order in
//    which codes are unpacked.
//  * Unpack with fp16 "magic numbers": OR-ing a code field into the mantissa
//    of fp16 1024.0 gives 1024 + m*code exactly (m = 1, 4, 16, 64 or 256 by
//    the field's bit position), two weights per 32-bit register, one
//    v_and_or_b32 each, ready for v_dot2_f32_f16 (fp16 products, fp32
//    accumulation).  The constant 1024*x part is removed per chunk by
//    subtracting the same dot-product chain evaluated on zero-point codes, so
//    groups whose codes all equal the zero point contribute exactly 0.
//  * Per-group fp16 scale (and int4 zero) are applied once per chunk in fp32;
//    the row sum is a DPP butterfly inside the lane group; fp16 y is rounded
//    to nearest even.  The binary coding XORs code and x words and counts
//    bits (v_bcnt_u32_b32): y = K - 2 * popcount (Whetstone README, "Measured
//    hardware facts").
//  * Greedy selection (a separate kernel variant): the workgroups of one
//    chosen matrix also reduce their outputs, in registers, to the largest
//    (value, smallest row) as a 64-bit order-preserving key and store it to
//    their own slot of a caller scratch array; a one-workgroup kernel then
//    reduces the slots to the winning row, so the index of the largest logit
//    never goes through the host and the logits are not read back (Whetstone
//    README, status list: the greedy path stays on the GPU).  Slots instead
//    of atomics: the output projection's tiles finish together at the end of
//    a sweep, and thousands of device-scope atomics on one address serialise.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace tkq {

namespace {

// Codings (bit fmt) whose runner keeps two load buffers, the next row steps'
// loads in flight while the current ones are computed (measured per coding:
// 1-2 % faster for K5 and binary; slower for ternary, int2, int3 and the
// greedy variant and equal for hier-g32, which keep one buffer and more
// waves).  int4 g128 has a kernel of its own (gemv_int4_kernel below).
constexpr int kPingpongMask = (1 << kFmtK5) | (1 << kFmtBin);
// Codings (bit fmt) whose code loads are plain rather than non-temporal.
// Binary rows (K/8 bytes) start at 32 bytes past a 64-byte boundary on odd
// rows, and a row's passes end mid-block: blocks touched by two load
// instructions were fetched from HBM twice under the non-temporal hint
// (traffic 1.080x against 1.002x plain; plain loads measured 3.89 -> 4.63
// TB/s on the binary shapes).  Ternary and int2 measured 5 % slower plain.
constexpr int kPlainMask = 1 << kFmtBin;
// Codings (bit fmt) whose waves raise their priority while issuing a row
// step's loads, so that a CU's loads are not held behind other waves' unpack
// work: int4-hier-g32 (+1.9 %); K5 -2 %, ternary -4 %, int3 -3 %, binary
// +0.5 %.
constexpr int kSetprioMask = 1 << kFmtHier;

constexpr int kWaves = 4;
constexpr int kMaxTileRows = kGemvMaxTileRows;
static_assert(sizeof(tkq_gemv_desc) == 64, "descriptor layout");
constexpr uint32_t kMagic = 0x64006400u;  // fp16 pair (1024.0, 1024.0)

// Constants held in registers.  A gfx9 VOP3 instruction (v_and_or_b32,
// v_perm_b32) can encode no literal and read at most one SGPR, so masks live
// in SGPRs and the magic number in a VGPR; the opaque moves keep the compiler
// from folding them back into literals.
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

// ---------------------------------------------------------------- codecs --
// Each codec states, for one 16-byte chunk of codes:
//   WPC  weights per chunk
//   PLANES  16-byte loads per chunk (one per plane of the matrix)
//   XR   u32 registers of prepared x (pairs of fp16)
//   XB   bytes of x the chunk consumes
//   CPG  chunks per 128-weight group;  MB metadata bytes per group
//   Regs register-resident constants (make() once per tile)
//   Sub  the fp16 pairs subtracted from the unpacked codes: 1024 + m * zero
//        for every multiplier class m of the chunk (sub(meta) per chunk)
//   prep(raw, xr)          permute natural x pairs into the unpack order
//   dot(codes, xr, R, S)   sum over the chunk of m * (code - zero) * x, as fp32
//
// The unpack ORs a code field into the mantissa of fp16 1024.0, giving
// 1024 + m * code exactly; subtracting 1024 + m * zero in fp16 is exact too
// (both are integers below 2048), so each v_dot2_f32_f16 multiplies x by a
// small exact integer and the fp32 sums carry only the weights' own terms.
// (Summing (1024 + m code) x and removing 1024 x afterwards leaves a rounding
// error that grows with 1024 |x| rather than with |w x|: large activation
// channels on weights at their zero point pushed it past the tolerance.)

template <int FMT>
struct Codec;

__device__ __forceinline__ h2 bcast_hi(uint32_t m) {  // (hi half, hi half)
  const _Float16 z = as_h2(m)[1];
  return (h2){z, z};
}
__device__ __forceinline__ h2 h2c(float v) { return (h2){(_Float16)v, (_Float16)v}; }

// int4: word w holds nibbles q0..q7 of elements 8i..8i+7.  (w & 0x000F000F)
// pairs (q0, q4); (w & 0x00F000F0) pairs (16 q1, 16 q5); the same on w >> 8
// gives (q2, q6) and (16 q3, 16 q7).  Two accumulators keep the x16 fields
// apart and are combined as lo + hi/16.
template <>
struct Codec<kFmtInt4> {
  static constexpr int WPC = 32, XR = 16, XB = 64, CPG = 4, MB = 4, PLANES = 1;
  struct Regs {
    uint32_t m0, m1, magic;
  };
  struct Sub {
    h2 c1, c16;
  };
  __device__ static Regs make() { return {in_sgpr(0x000F000Fu), in_sgpr(0x00F000F0u), in_vgpr(kMagic)}; }
  // (1024 + z, 1024 + 16 z) from the group's half2 {scale, zero}
  __device__ static Sub sub(uint32_t meta, const Regs& R) {
    const h2 zz = bcast_hi(meta), mg = as_h2(R.magic);
    return {zz + mg, zz * h2c(16.0f) + mg};
  }
  __device__ static void prep(const uint32_t* raw, uint32_t* xr) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = raw[4 * w], b = raw[4 * w + 1], c = raw[4 * w + 2], d = raw[4 * w + 3];
      xr[4 * w + 0] = __builtin_amdgcn_perm(c, a, 0x05040100u);  // (x0, x4)
      xr[4 * w + 1] = __builtin_amdgcn_perm(c, a, 0x07060302u);  // (x1, x5)
      xr[4 * w + 2] = __builtin_amdgcn_perm(d, b, 0x05040100u);  // (x2, x6)
      xr[4 * w + 3] = __builtin_amdgcn_perm(d, b, 0x07060302u);  // (x3, x7)
    }
  }
  __device__ static float dot(u32x4 q, const uint32_t* xr, const Regs& R, const Sub& S) {
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t v = q[w], t = v >> 8;
      lo = __builtin_amdgcn_fdot2(as_h2((v & R.m0) | R.magic) - S.c1, as_h2(xr[4 * w + 0]), lo, false);
      hi = __builtin_amdgcn_fdot2(as_h2((v & R.m1) | R.magic) - S.c16, as_h2(xr[4 * w + 1]), hi, false);
      lo = __builtin_amdgcn_fdot2(as_h2((t & R.m0) | R.magic) - S.c1, as_h2(xr[4 * w + 2]), lo, false);
      hi = __builtin_amdgcn_fdot2(as_h2((t & R.m1) | R.magic) - S.c16, as_h2(xr[4 * w + 3]), hi, false);
    }
    return fmaf(hi, 0.0625f, lo);
  }
};

// K5: one byte per weight.  v_perm builds (1024 + c0, 1024 + c2) and
// (1024 + c1, 1024 + c3) from a code word and the byte 0x64; the pair
// (1145, 1145) = 1024 + 121 is subtracted (byte 121 = value 0).
template <>
struct Codec<kFmtK5> {
  static constexpr int WPC = 16, XR = 8, XB = 32, CPG = 8, MB = 2, PLANES = 1;
  struct Regs {
    uint32_t sel_a, sel_b, magic, zero;
  };
  struct Sub {};
  __device__ static Regs make() {
    return {in_sgpr(0x04020400u), in_sgpr(0x04030401u), in_vgpr(0x64646464u), in_sgpr(0x64796479u)};
  }
  __device__ static Sub sub(uint32_t, const Regs&) { return {}; }
  __device__ static void prep(const uint32_t* raw, uint32_t* xr) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = raw[2 * w], b = raw[2 * w + 1];  // (x0,x1), (x2,x3)
      xr[2 * w + 0] = __builtin_amdgcn_perm(b, a, 0x05040100u);  // (x0, x2)
      xr[2 * w + 1] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // (x1, x3)
    }
  }
  __device__ static float dot(u32x4 q, const uint32_t* xr, const Regs& R, const Sub&) {
    float acc = 0.0f;
    const h2 z = as_h2(R.zero);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t v = q[w];
      acc = __builtin_amdgcn_fdot2(as_h2(__builtin_amdgcn_perm(R.magic, v, R.sel_a)) - z, as_h2(xr[2 * w + 0]),
                                   acc, false);
      acc = __builtin_amdgcn_fdot2(as_h2(__builtin_amdgcn_perm(R.magic, v, R.sel_b)) - z, as_h2(xr[2 * w + 1]),
                                   acc, false);
    }
    return acc;
  }
};

// 2-bit fields (ternary and int2), element 16i+s at bits 2s.  Masks 3 << 2s
// for s = 0..4 (both halves) give (1024 + 4^s c_s, 1024 + 4^s c_{s+8}); the
// word shifted right by 10 gives s = 5, 6, 7 with multipliers 1, 4, 16.  The
// five multiplier classes subtract c[0..4] = 1024 + 4^s * zero.
struct Sub2 {
  h2 c[5];
};
struct Regs2 {
  uint32_t m[5], magic;
};
__device__ __forceinline__ Regs2 make2() {
  return {{in_sgpr(0x00030003u), in_sgpr(0x000C000Cu), in_sgpr(0x00300030u), in_sgpr(0x00C000C0u),
           in_sgpr(0x03000300u)},
          in_vgpr(kMagic)};
}
__device__ __forceinline__ void prep2(const uint32_t* raw, uint32_t* xr) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // raw[8w + p] = (x_{2p}, x_{2p+1}) of word w's 16 elements
    const uint32_t* r = raw + 8 * w;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t lo = r[s >> 1], hi = r[4 + (s >> 1)];
      xr[8 * w + s] = (s & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                              : __builtin_amdgcn_perm(hi, lo, 0x05040100u);  // (x_s, x_{s+8})
    }
  }
}
__device__ __forceinline__ float dot2bit(u32x4 q, const uint32_t* xr, const Regs2& R, const Sub2& S) {
  float a1 = 0.0f, a4 = 0.0f, a16 = 0.0f, a64 = 0.0f, a256 = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t v = q[w], t = v >> 10;
    const uint32_t* x = xr + 8 * w;
    a1 = __builtin_amdgcn_fdot2(as_h2((v & R.m[0]) | R.magic) - S.c[0], as_h2(x[0]), a1, false);
    a4 = __builtin_amdgcn_fdot2(as_h2((v & R.m[1]) | R.magic) - S.c[1], as_h2(x[1]), a4, false);
    a16 = __builtin_amdgcn_fdot2(as_h2((v & R.m[2]) | R.magic) - S.c[2], as_h2(x[2]), a16, false);
    a64 = __builtin_amdgcn_fdot2(as_h2((v & R.m[3]) | R.magic) - S.c[3], as_h2(x[3]), a64, false);
    a256 = __builtin_amdgcn_fdot2(as_h2((v & R.m[4]) | R.magic) - S.c[4], as_h2(x[4]), a256, false);
    a1 = __builtin_amdgcn_fdot2(as_h2((t & R.m[0]) | R.magic) - S.c[0], as_h2(x[5]), a1, false);
    a4 = __builtin_amdgcn_fdot2(as_h2((t & R.m[1]) | R.magic) - S.c[1], as_h2(x[6]), a4, false);
    a16 = __builtin_amdgcn_fdot2(as_h2((t & R.m[2]) | R.magic) - S.c[2], as_h2(x[7]), a16, false);
  }
  return fmaf(a256, 0.00390625f, fmaf(a64, 0.015625f, fmaf(a16, 0.0625f, fmaf(a4, 0.25f, a1))));
}

// Ternary: code = t + 1, so the zero code is 1 in every field.
template <>
struct Codec<kFmtTern> {
  static constexpr int WPC = 64, XR = 32, XB = 128, CPG = 2, MB = 2, PLANES = 1;
  using Regs = Regs2;
  using Sub = Sub2;
  __device__ static Regs make() { return make2(); }
  __device__ static Sub sub(uint32_t, const Regs&) {
    return {{h2c(1025.0f), h2c(1028.0f), h2c(1040.0f), h2c(1088.0f), h2c(1280.0f)}};
  }
  __device__ static void prep(const uint32_t* raw, uint32_t* xr) { prep2(raw, xr); }
  __device__ static float dot(u32x4 q, const uint32_t* xr, const Regs& R, const Sub& S) {
    return dot2bit(q, xr, R, S);
  }
};

// int4-hier-g32: the int4 code layout, so the int4 unpack with 1024 removed
// from both fields (the dot is sum q x); a chunk is exactly one 32-weight
// group, whose metadata is one byte (scale index | min index << 4).  The
// row's fp16 pair (d, dmin) is applied once per row.
template <>
struct Codec<kFmtHier> : Codec<kFmtInt4> {
  static constexpr int CPG = 1, MB = 1;
  __device__ static Sub sub(uint32_t, const Regs& R) { return {as_h2(R.magic), as_h2(R.magic)}; }
};

// int2 g128: the ternary field layout and the int4 metadata (fp16 scale and
// zero-point), so c[s] = 1024 + 4^s z per group.
template <>
struct Codec<kFmtInt2> {
  static constexpr int WPC = 64, XR = 32, XB = 128, CPG = 2, MB = 4, PLANES = 1;
  using Regs = Regs2;
  using Sub = Sub2;
  __device__ static Regs make() { return make2(); }
  __device__ static Sub sub(uint32_t meta, const Regs& R) {
    const h2 zz = bcast_hi(meta), mg = as_h2(R.magic);
    return {{zz + mg, zz * h2c(4.0f) + mg, zz * h2c(16.0f) + mg, zz * h2c(64.0f) + mg, zz * h2c(256.0f) + mg}};
  }
  __device__ static void prep(const uint32_t* raw, uint32_t* xr) { prep2(raw, xr); }
  __device__ static float dot(u32x4 q, const uint32_t* xr, const Regs& R, const Sub& S) {
    return dot2bit(q, xr, R, S);
  }
};

// int3 g128: a chunk is one 128-group = three 16-byte planes (12 words, four
// 32-weight blocks of three words).  Word j of a block holds codes 10j..10j+4
// at bits 3f and 10j+5..10j+9 at bits 16+3f, so masks 7<<3f on both halves
// give (1024 + 8^f c, 1024 + 8^f c') for f = 0, 1, 2 and the word shifted
// right by 9 gives f = 3, 4 with multipliers 1, 8.  Codes 30 and 31 are
// spread over bits 15 and 31 of the three words (bit j in word j) and are
// gathered into one pair with three shift + and_or steps.  Metadata as int4;
// the classes subtract 1024 + z, 1024 + 8 z and 1024 + 64 z.
// The planes are matrix-wide (plane p of row n at byte p*N*K/8 + n*K/8), so a
// row step's load of one plane covers consecutive rows without gaps: with
// planes interleaved per row, the 32-byte sectors at plane boundaries were
// shared by two load instructions and, under the non-temporal hint, fetched
// from HBM twice (11 % more traffic on the 0.5B sweep).
struct Planes3 {
  u32x4 p[3];
};

template <>
struct Codec<kFmtInt3> {
  static constexpr int WPC = 128, XR = 64, XB = 256, CPG = 1, MB = 4, PLANES = 3;
  struct Regs {
    uint32_t m0, m1, m2, s0, s1, s2, magic;
  };
  struct Sub {
    h2 c1, c8, c64;
  };
  __device__ static Regs make() {
    return {in_sgpr(0x00070007u), in_sgpr(0x00380038u), in_sgpr(0x01C001C0u), in_sgpr(0x00010001u),
            in_sgpr(0x00020002u), in_sgpr(0x00040004u), in_vgpr(kMagic)};
  }
  __device__ static Sub sub(uint32_t meta, const Regs& R) {
    const h2 zz = bcast_hi(meta), mg = as_h2(R.magic);
    return {zz + mg, zz * h2c(8.0f) + mg, zz * h2c(64.0f) + mg};
  }
  // pair (e1, e2) of a block's x values; raw[i] = (x_2i, x_2i+1)
  __device__ static uint32_t xpair(const uint32_t* raw, int e1, int e2) {
    const uint32_t lo = (e1 & 1) ? 0x0302u : 0x0100u, hi = (e2 & 1) ? 0x0706u : 0x0504u;
    return __builtin_amdgcn_perm(raw[e2 >> 1], raw[e1 >> 1], (hi << 16) | lo);
  }
  __device__ static void prep(const uint32_t* raw, uint32_t* xr) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t* r = raw + 16 * b;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
#pragma unroll
        for (int f = 0; f < 5; ++f) xr[16 * b + 5 * j + f] = xpair(r, 10 * j + f, 10 * j + 5 + f);
      }
      xr[16 * b + 15] = xpair(r, 30, 31);
    }
  }
  __device__ static float dot(const Planes3& q, const uint32_t* xr, const Regs& R, const Sub& S) {
    float a1 = 0.0f, a8 = 0.0f, a64 = 0.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      uint32_t w[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int n = 3 * b + j;
        w[j] = q.p[n >> 2][n & 3];
      }
      const uint32_t* x = xr + 16 * b;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const uint32_t v = w[j], t = v >> 9;
        a1 = __builtin_amdgcn_fdot2(as_h2((v & R.m0) | R.magic) - S.c1, as_h2(x[5 * j + 0]), a1, false);
        a8 = __builtin_amdgcn_fdot2(as_h2((v & R.m1) | R.magic) - S.c8, as_h2(x[5 * j + 1]), a8, false);
        a64 = __builtin_amdgcn_fdot2(as_h2((v & R.m2) | R.magic) - S.c64, as_h2(x[5 * j + 2]), a64, false);
        a1 = __builtin_amdgcn_fdot2(as_h2((t & R.m0) | R.magic) - S.c1, as_h2(x[5 * j + 3]), a1, false);
        a8 = __builtin_amdgcn_fdot2(as_h2((t & R.m1) | R.magic) - S.c8, as_h2(x[5 * j + 4]), a8, false);
      }
      uint32_t p = ((w[0] >> 15) & R.s0) | R.magic;
      p = ((w[1] >> 14) & R.s1) | p;
      p = ((w[2] >> 13) & R.s2) | p;
      a1 = __builtin_amdgcn_fdot2(as_h2(p) - S.c1, as_h2(x[15]), a1, false);
    }
    return fmaf(a64, 0.015625f, fmaf(a8, 0.125f, a1));
  }
};

// Binary: 128 sign bits per chunk; x is kept as packed words.
template <>
struct Codec<kFmtBin> {
  static constexpr int WPC = 128, XR = 4, XB = 16, CPG = 1, MB = 0, PLANES = 1;
  struct Regs {};
  struct Sub {};
  __device__ static Regs make() { return {}; }
  __device__ static Sub sub(uint32_t, const Regs&) { return {}; }
  __device__ static void prep(const uint32_t* raw, uint32_t* xr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[i] = raw[i];
  }
  __device__ static int dot(u32x4 q, const uint32_t* xr, const Regs&, const Sub&) {
    int acc = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc += __builtin_popcount(q[w] ^ xr[w]);
    return acc;
  }
};

// ------------------------------------------------------------ tile runner --
struct Tile {
  __amdgpu_buffer_rsrc_t codes, meta, x, y;
  __amdgpu_buffer_rsrc_t rmeta;  // int4-hier-g32: the rows' fp16 (d, dmin) pairs
  __amdgpu_buffer_rsrc_t codes_p1, codes_p2;  // int3: the tile's rows in planes 1 and 2
  uint32_t row_bytes;       // bytes of codes per row (of one plane for int3)
  size_t plane_stride;      // int3: bytes from one plane of the matrix to the next
  uint32_t meta_row_bytes;  // bytes of metadata per row
  int lg, sub, prow, P;     // lanes-per-row log2, lane in group, row in step, rows per step
  int S, slice;             // k-slices, this wave's slice
  int rbase, steps;         // first tile row of this wave, row steps
  int Cs, C, K;             // chunks per slice, chunks per row, columns
  int row0, nrows;          // first matrix row of the tile, rows in the tile
  bool track;               // greedy selection over this matrix
  // wave-uniform bases of the tile's codes and metadata: each row step gets a
  // buffer resource that starts at its first row (scalar arithmetic), so the
  // per-lane offsets stay loop-invariant and the range check stays exact
  const char* codes_ptr;
  const char* meta_ptr;
  uint32_t codes_bytes, meta_bytes;
};

// Codings (bit fmt) whose loads use per-step scalar bases (measured per
// coding: faster for hier-g32, slower for ternary and K5).
constexpr int kSbaseMask = 1 << kFmtHier;

// Order-preserving key of an output: larger value -> larger key, and among
// equal values the smaller row -> larger key.  fp16: -0 counts as +0, and
// every NaN (either sign, any payload) counts as larger than +inf, so the
// first NaN wins (numpy's argmax convention); int32 (binary): two's
// complement.
__device__ __forceinline__ uint64_t greedy_key_f16(uint32_t bits, uint32_t row) {
  bits &= 0xFFFFu;
  if (bits == 0x8000u) bits = 0u;
  uint32_t ord = (bits & 0x8000u) ? (~bits & 0xFFFFu) : (bits | 0x8000u);
  if ((bits & 0x7FFFu) > 0x7C00u) ord = 0xFFFFu;  // NaN
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - row);
}
__device__ __forceinline__ uint64_t greedy_key_i32(uint32_t v, uint32_t row) {
  return ((uint64_t)(v ^ 0x80000000u) << 32) | (uint64_t)(0xFFFFFFFFu - row);
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
// Whole-wave maximum in every lane without the LDS pipe: DPP quad and mirror
// steps within rows of 16 lanes, then gfx950's permlane swaps across rows
// (with the value in both operands the two results hold each lane's own
// value and that of lane ^ 16 or ^ 32).
template <int CTRL>
__device__ __forceinline__ uint64_t max_dpp_u64(uint64_t v) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(v >> 32), CTRL, 0xF, 0xF, false);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  return max_u64(v, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint64_t max_swap_u64(uint64_t v, bool wide) {
  const uint32_t h = (uint32_t)(v >> 32), l = (uint32_t)v;
  const auto rh = wide ? __builtin_amdgcn_permlane32_swap(h, h, false, false)
                       : __builtin_amdgcn_permlane16_swap(h, h, false, false);
  const auto rl = wide ? __builtin_amdgcn_permlane32_swap(l, l, false, false)
                       : __builtin_amdgcn_permlane16_swap(l, l, false, false);
  return max_u64(((uint64_t)rh[0] << 32) | rl[0], ((uint64_t)rh[1] << 32) | rl[1]);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_dpp_u64<kQuadSwap1>(v);
  v = max_dpp_u64<kQuadSwap2>(v);
  v = max_dpp_u64<kRowHalfMirror>(v);
  v = max_dpp_u64<kRowMirror>(v);
  return max_swap_u64(max_swap_u64(v, false), true);
}

constexpr uint32_t kFar = 0x80000000u;  // offset past any buffer, no wrap

template <int FMT, int J, int U, bool GREEDY>
struct Runner {
  using Cd = Codec<FMT>;
  static constexpr bool kBin = FMT == kFmtBin;
  using Acc = typename std::conditional<kBin, int, float>::type;

  using Chunk = typename std::conditional<Cd::PLANES == 3, Planes3, u32x4>::type;
  struct Buf {
    Chunk c[U][J];
    uint32_t m[U][J];
    uint32_t rp[U];  // int4-hier-g32 row pair
  };

  const Tile& t;
  typename Cd::Regs R;
  uint32_t cof[J], mof[J];
  uint32_t vc[J], vm[J];  // cof / mof plus this lane's row within a step
  uint32_t xr[J][Cd::XR];
  float xsum[FMT == kFmtHier ? J : 1];  // int4-hier-g32: sum of each chunk's x
  mutable uint64_t best = 0;  // greedy variant: best key of this lane's rows

  __device__ __forceinline__ Runner(const Tile& tile) : t(tile), R(Cd::make()) {
    // Fixed chunk positions of this lane.
    const int L = 1 << t.lg;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int local = t.sub + L * j;  // lane `sub` of the row's L lanes reads chunks sub, sub + L, ...
      const int c = t.slice * t.Cs + local;
      const bool ok = local < t.Cs && c < t.C;
      cof[j] = ok ? (uint32_t)c * 16u : kFar;
      mof[j] = ok ? (uint32_t)(c / Cd::CPG) * Cd::MB : kFar;
      vc[j] = ok ? (uint32_t)t.prow * t.row_bytes + cof[j] : kFar;
      vm[j] = ok ? (uint32_t)t.prow * t.meta_row_bytes + mof[j] : kFar;
    }
  }

  // This lane's slice of x, permuted for the unpack, and its constants.
  __device__ __forceinline__ void load_x() {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t xo = cof[j] == kFar ? kFar : (cof[j] / 16u) * (uint32_t)Cd::XB;
      uint32_t raw[Cd::XR];
#pragma unroll
      for (int i = 0; i < Cd::XR / 4; ++i) {
        const u32x4 v = load16(t.x, xo == kFar ? kFar : xo + 16u * i);
        raw[4 * i + 0] = v[0];
        raw[4 * i + 1] = v[1];
        raw[4 * i + 2] = v[2];
        raw[4 * i + 3] = v[3];
      }
      Cd::prep(raw, xr[j]);
      if constexpr (FMT == kFmtHier) {  // sum of the chunk's x, for the min term
        float sx = 0.0f;
#pragma unroll
        for (int i = 0; i < Cd::XR; ++i) sx = __builtin_amdgcn_fdot2(as_h2(xr[j][i]), as_h2(0x3C003C00u), sx, false);
        xsum[j] = sx;
      }
    }
  }

  __device__ __forceinline__ uint32_t row(int st, int u) const {
    return (uint32_t)(t.rbase + (st + u) * t.P + t.prow);
  }

  static constexpr bool kSbase = (kSbaseMask >> FMT) & 1;
  static constexpr bool kPlain = (kPlainMask >> FMT) & 1;
  __device__ static __forceinline__ u32x4 code16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return kPlain ? load16(r, off) : load16_nt(r, off);
  }

  static constexpr bool kSetprio = (kSetprioMask >> FMT) & 1;
  __device__ __forceinline__ void issue(int st, Buf& b) const {
    if constexpr (kSetprio) __builtin_amdgcn_s_setprio(1);
    issue_loads(st, b);
    if constexpr (kSetprio) __builtin_amdgcn_s_setprio(0);
  }
  __device__ __forceinline__ void issue_loads(int st, Buf& b) const {
    if constexpr (kSbase) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t s = (uint32_t)(t.rbase + (st + u) * t.P);  // first row of the step (uniform)
      const __amdgpu_buffer_rsrc_t rc = make_rsrc_uniform(t.codes_ptr, s * t.row_bytes, t.codes_bytes);
      const __amdgpu_buffer_rsrc_t rm = make_rsrc_uniform(t.meta_ptr, s * t.meta_row_bytes, t.meta_bytes);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if constexpr (Cd::PLANES == 3) {
#pragma unroll
          for (int p = 0; p < 3; ++p)
            b.c[u][j].p[p] = code16(
                make_rsrc_uniform(t.codes_ptr + p * t.plane_stride, s * t.row_bytes, t.codes_bytes), vc[j]);
        } else {
          b.c[u][j] = code16(rc, vc[j]);
        }
        if constexpr (Cd::MB == 4) b.m[u][j] = load4(rm, vm[j]);
        else if constexpr (Cd::MB == 2) b.m[u][j] = load2(rm, vm[j]);
        else if constexpr (Cd::MB == 1) b.m[u][j] = load1(rm, vm[j]);
        else b.m[u][j] = 0;
      }
      if constexpr (FMT == kFmtHier) b.rp[u] = load4(t.rmeta, row(st, u) * 4u);
    }
    } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t r = row(st, u);
      const uint32_t rb = r * t.row_bytes, mb = r * t.meta_row_bytes;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if constexpr (Cd::PLANES == 3) {
          b.c[u][j].p[0] = code16(t.codes, rb + cof[j]);
          b.c[u][j].p[1] = code16(t.codes_p1, rb + cof[j]);
          b.c[u][j].p[2] = code16(t.codes_p2, rb + cof[j]);
        } else {
          b.c[u][j] = code16(t.codes, rb + cof[j]);
        }
        if constexpr (Cd::MB == 4) b.m[u][j] = load4(t.meta, mb + mof[j]);
        else if constexpr (Cd::MB == 2) b.m[u][j] = load2(t.meta, mb + mof[j]);
        else if constexpr (Cd::MB == 1) b.m[u][j] = load1(t.meta, mb + mof[j]);
        else b.m[u][j] = 0;
      }
      if constexpr (FMT == kFmtHier) b.rp[u] = load4(t.rmeta, r * 4u);
    }
    }
  }

  // One row step's output value of this lane -> y (or the k-slice partials).
  __device__ __forceinline__ void finish(int st, int u, float fv, int iv, bool writer, uint32_t* part) const {
    const uint32_t r = row(st, u);
    if (!writer) return;
    if (t.S == 1) {
      if constexpr (kBin) {
        const uint32_t o = (uint32_t)(t.K - 2 * iv);
        store4(t.y, r * 4u, o);
        if (GREEDY && t.track && r < (uint32_t)t.nrows) best = max_u64(best, greedy_key_i32(o, t.row0 + r));
      } else {
        const uint16_t h = half_bits(fv);
        store2(t.y, r * 2u, h);
        if (GREEDY && t.track && r < (uint32_t)t.nrows) best = max_u64(best, greedy_key_f16(h, t.row0 + r));
      }
    } else if (r < (uint32_t)kMaxTileRows) {
      part[t.slice * kMaxTileRows + r] = kBin ? (uint32_t)iv : u32(fv);
    }
  }

  __device__ __forceinline__ void compute(int st, const Buf& b, uint32_t* part) const {
    const int L = 1 << t.lg;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Acc res = 0;
      float rs = 0.0f, rm = 0.0f;  // int4-hier-g32: sum of sc*dot, sum of mi*sum(x)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint32_t m = b.m[u][j];
        if constexpr (kBin) {
          res += Cd::dot(b.c[u][j], xr[j], R, typename Cd::Sub{});
        } else if constexpr (FMT == kFmtHier) {
          const float d = Cd::dot(b.c[u][j], xr[j], R, Cd::sub(m, R));  // sum q x
          rs = fmaf((float)(m & 15u), d, rs);
          rm = fmaf((float)(m >> 4), xsum[j], rm);
        } else {  // sum (q - z) x, times the group scale (low half of the metadata)
          const float d = Cd::dot(b.c[u][j], xr[j], R, Cd::sub(m, R));
          res = fmaf(half_lo(m), d, res);
        }
      }
      if constexpr (FMT == kFmtHier) res = fmaf(half_lo(b.rp[u]), rs, -half_hi(b.rp[u]) * rm);
      const Acc v = group_sum(res, t.lg);
      if constexpr (kBin) finish(st, u, 0.0f, v, t.sub == L - 1, part);
      else finish(st, u, v, 0, t.sub == L - 1, part);
    }
  }

  static constexpr bool kPingpong = ((kPingpongMask >> FMT) & 1) && !GREEDY;

  __device__ __forceinline__ void run(uint32_t* part) {
    if constexpr (kPingpong) {
      // Two buffers used alternately: the loads of step st + U are in flight
      // while step st is computed.
      Buf a, b;
      issue(0, a);  // the first codes stream in while x is prepared
      load_x();
      for (int st = 0; st < t.steps; st += 2 * U) {
        if (st + U < t.steps) issue(st + U, b);
        compute(st, a, part);
        if (st + U >= t.steps) break;
        if (st + 2 * U < t.steps) issue(st + 2 * U, a);
        compute(st + U, b, part);
      }
    } else {
      // One buffer: U row steps are loaded, then computed; the other waves of
      // the CU keep the memory system busy meanwhile.
      Buf a;
      issue(0, a);  // the first codes stream in while x is prepared
      load_x();
      for (int st = 0; st < t.steps; st += U) {
        if (st > 0) issue(st, a);
        compute(st, a, part);
      }
    }
  }
};

// Row steps per loop iteration: the planner's unroll, or for the 48-byte
// int3 chunks a divisor of it (tile heights stay multiples).
constexpr int kInt3Unroll = 2;
template <int FMT, int J>
constexpr int runner_unroll() {
  return Codec<FMT>::PLANES == 3 ? (gemv_unroll(J) % kInt3Unroll == 0 ? kInt3Unroll : 1) : gemv_unroll(J);
}

template <int FMT, int J, bool GREEDY>
__device__ __forceinline__ uint64_t run_passes(const Tile& t, uint32_t* part) {
  Runner<FMT, J, runner_unroll<FMT, J>(), GREEDY> r(t);
  r.run(part);
  return r.best;
}

// ------------------------------------------------------------------ kernel --
// JMAX: the largest pass count among the launch's descriptors; only the
// cases up to it are instantiated, so registers match the workload.
// Greedy variant arguments: the target descriptor and the slot array (one
// key per tile of the target).
struct Greedy {
  int target;
  uint64_t* slots;
};

template <int FMT, int JMAX, bool GREEDY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 8))) void gemv_kernel(
    const tkq_gemv_desc* __restrict__ descs, int count, Greedy g) {
  using Cd = Codec<FMT>;
  constexpr bool kBin = FMT == kFmtBin;
  __shared__ uint32_t part[kWaves * kMaxTileRows];
  __shared__ unsigned long long wave_best[kWaves];

  // The matrix this workgroup works on: last descriptor with work0 <= tile
  // (binary search; the loads hit the scalar cache after the first few).
  const int tile = blockIdx.x;
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (descs[mid].work0 <= tile) lo = mid;
    else hi = mid - 1;
  }
  const tkq_gemv_desc* d = descs + lo;
  const int N = d->N, K = d->K;
  // Large tiles first, then small tiles for the rest of the matrix.
  const int local = tile - d->work0, nbig = d->big_tiles;
  const int rpt = local < nbig ? d->rows_per_tile : d->small_rows;
  const int row0 = local < nbig ? local * rpt : nbig * d->rows_per_tile + (local - nbig) * rpt;
  const GemvShape sh = unpack_shape(d->shape);

  Tile t;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  t.lg = sh.lanes_log2;
  t.P = 64 >> t.lg;
  t.sub = lane & ((1 << t.lg) - 1);
  t.prow = lane >> t.lg;
  t.S = sh.kslices;
  t.slice = wave & (t.S - 1);
  const int rg = wave / t.S, rows_per_rg = rpt / (kWaves / t.S);
  t.rbase = rg * rows_per_rg;
  t.steps = rows_per_rg / t.P;
  t.K = K;
  t.C = K / Cd::WPC;
  t.Cs = (t.C + t.S - 1) / t.S;
  t.row_bytes = (uint32_t)t.C * 16u;
  t.meta_row_bytes = (uint32_t)(t.C / Cd::CPG) * Cd::MB;
  const int nrows = min(rpt, N - row0);
  t.row0 = row0;
  t.nrows = nrows;
  t.track = GREEDY && lo == g.target;
  const char* codes = (const char*)d->codes + (size_t)row0 * t.row_bytes;
  t.codes = make_rsrc(codes, (uint32_t)nrows * t.row_bytes);
  t.codes_ptr = codes;
  t.codes_bytes = (uint32_t)nrows * t.row_bytes;
  t.plane_stride = (size_t)N * t.row_bytes;
  if constexpr (Cd::PLANES == 3) {
    t.codes_p1 = make_rsrc(codes + t.plane_stride, t.codes_bytes);
    t.codes_p2 = make_rsrc(codes + 2 * t.plane_stride, t.codes_bytes);
  } else {
    t.codes_p1 = t.codes_p2 = t.codes;
  }
  if constexpr (Cd::MB > 0) {
    const char* meta = (const char*)d->meta + (size_t)row0 * t.meta_row_bytes;
    t.meta = make_rsrc(meta, (uint32_t)nrows * t.meta_row_bytes);
    t.meta_ptr = meta;
    t.meta_bytes = (uint32_t)nrows * t.meta_row_bytes;
  } else {
    t.meta = make_rsrc(d->codes, 0u);
    t.meta_ptr = (const char*)d->codes;
    t.meta_bytes = 0u;
  }
  if constexpr (FMT == kFmtHier) {
    const char* rm = (const char*)d->meta + hier_row_offset(N, K) + (size_t)row0 * 4u;
    t.rmeta = make_rsrc(rm, (uint32_t)nrows * 4u);
  } else {
    t.rmeta = t.meta;
  }
  t.x = make_rsrc(d->x, kBin ? (uint32_t)(K / 8) : (uint32_t)K * 2u);
  const uint32_t ybytes = kBin ? 4u : 2u;
  t.y = make_rsrc((char*)d->y + (size_t)row0 * ybytes, (uint32_t)nrows * ybytes);

  uint64_t best = 0;
  switch (sh.passes) {
#define TKQ_CASE(J)                                                \
  case J:                                                          \
    if constexpr (J <= JMAX) best = run_passes<FMT, J, GREEDY>(t, part); \
    break;
    TKQ_CASE(1)
    TKQ_CASE(2)
    TKQ_CASE(3)
    TKQ_CASE(4)
    TKQ_CASE(5)
    TKQ_CASE(6)
    TKQ_CASE(7)
    TKQ_CASE(8)
#undef TKQ_CASE
    default: break;
  }

  if (t.S > 1) {
    __syncthreads();
    for (int r = threadIdx.x; r < nrows && r < kMaxTileRows; r += 64 * kWaves) {
      if constexpr (kBin) {
        int v = 0;
        for (int s = 0; s < t.S; ++s) v += (int)part[s * kMaxTileRows + r];
        const uint32_t o = (uint32_t)(K - 2 * v);
        store4(t.y, (uint32_t)r * 4u, o);
        if (GREEDY && t.track) best = max_u64(best, greedy_key_i32(o, (uint32_t)(row0 + r)));
      } else {
        float v = 0.0f;
        for (int s = 0; s < t.S; ++s) v += f32(part[s * kMaxTileRows + r]);
        const uint16_t h = half_bits(v);
        store2(t.y, (uint32_t)r * 2u, h);
        if (GREEDY && t.track) best = max_u64(best, greedy_key_f16(h, (uint32_t)(row0 + r)));
      }
    }
  }

  if constexpr (GREEDY) {
    if (t.track) {  // uniform over the workgroup
      best = wave_max_u64(best);
      if (lane == 0) wave_best[wave] = best;
      __syncthreads();
      if (threadIdx.x == 0) {
        uint64_t b = wave_best[0];
        for (int w = 1; w < kWaves; ++w) b = max_u64(b, wave_best[w]);
        g.slots[tile - d->work0] = b;
      }
    }
  }
}

// ------------------------------------------------ int4 g128 stream kernel --
// The int4 g128 GEMV streams each tile's codes as 128-byte lines.  A tile of
// 32 R rows is cut into 32 units of R consecutive rows (8 lanes each, 8
// units per wave).  A unit walks its rows' 128-weight groups in memory order,
// two groups per pass: the lanes with an even index in the unit (quad 0)
// take the even group, the odd lanes (quad 1) the odd one, one 16-byte chunk
// per lane, so a pass reads 128 contiguous bytes of the unit's rows -- one
// whole cache line when rows start on 128-byte boundaries (K a multiple of
// 256, or R even) -- and every lane is busy for any K.  Both quads can be on
// different rows (odd groups per row), so each lane sums its quad's groups
// of a row on its own and, when the quad's next group starts a new row,
// writes that sum to the row's LDS slot for its lane (eight per row, written
// once each); the tile's rows are finished from their eight slots at the
// end, in a fixed order.
// Group metadata: every four passes each lane of a unit loads one word, the
// unit's next eight groups (32 contiguous bytes), and each pass hands its
// quad's word to the quad with one ds_swizzle.  x (permuted to the unpack
// order, 64 bytes per chunk; two copies back to back when the group count is
// odd, so that a pass's pair of groups is always adjacent) is staged in LDS
// while the first codes are in flight.  Codes flow through a register ring
// kInt4Depth passes deep, metadata two blocks (eight passes) ahead; the
// addresses of a pass are wave-uniform bases plus loop-invariant lane
// offsets.
//
// Unpack: the low nibble field of a half sits at mantissa bits 0-3, where
// fp16 1024.0 has ulp 1, and the high nibble field at bits 4-7, where fp16
// 64.0 has ulp 1/16; OR-ing the fields into those two constants gives
// 1024 + q and 64 + q exactly, and subtracting 1024 + z and 64 + z leaves
// q - z exactly in both, so one fp32 chain sums a chunk.
constexpr int kInt4Unroll = 8;                // passes per loop iteration: two metadata blocks
constexpr int kInt4Depth = 4;                 // passes of codes in flight per lane (divides kInt4Unroll)
constexpr uint32_t kMagic64 = 0x54005400u;   // fp16 pair (64.0, 64.0)

// ds_swizzle bit mode within 32 lanes: source lane = (lane & 0b11001) | 2j,
// i.e. unit lane 2j + q for every lane of quad q (j = pass within the block).
template <int J>
__device__ __forceinline__ uint32_t quad_meta(uint32_t words) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)words, 0x19 | ((2 * J) << 5));
}

template <bool GREEDY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 8))) void gemv_int4_kernel(
    const tkq_gemv_desc* __restrict__ descs, int count, Greedy g) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  __shared__ unsigned long long wave_best[kWaves];
  static_assert(kInt4Unroll == 8 && kInt4Unroll % kInt4Depth == 0, "two metadata blocks per iteration");

  const int tile = blockIdx.x;
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (descs[mid].work0 <= tile) lo = mid;
    else hi = mid - 1;
  }
  const tkq_gemv_desc* d = descs + lo;
  const int N = d->N, K = d->K;
  const int local = tile - d->work0, nbig = d->big_tiles;
  const int rpt = local < nbig ? d->rows_per_tile : d->small_rows;
  const int row0 = local < nbig ? local * rpt : nbig * d->rows_per_tile + (local - nbig) * rpt;
  const int nrows = min(rpt, N - row0);
  const bool track = GREEDY && lo == g.target;

  const int lane = threadIdx.x & 63;
  const int q = lane & 1, sub = (lane >> 1) & 3, ul = lane & 7;  // quad, lane in quad, lane in unit
  const int unit = (int)(threadIdx.x >> 3);             // 0..31
  const int G = K >> 7;                                  // groups per row
  const int R = rpt >> 5;                                // rows per unit
  const int RG = R * G, passes = (RG + 1) >> 1;
  const bool odd = (RG & 1) != 0;                        // quad 1 idle in the last pass
  const int xper = (G & 1) ? 2 * G : G;                  // groups of x held in LDS
  const uint32_t row_bytes = (uint32_t)K >> 1;
  uint32_t* xl = lds;                                    // 64 words per group
  float* pl = reinterpret_cast<float*>(lds + xper * 64);  // 8 partial slots per row

  // Codes: pass p of a unit reads bytes 128 p .. 128 p + 127 of the unit's
  // rows; metadata block B (passes 4B .. 4B + 3) is the unit's groups
  // 8B .. 8B + 7.  Loads past the unit's last pass get an empty range.
  const char* tcodes = (const char*)d->codes + (size_t)row0 * row_bytes;
  const char* tmeta = (const char*)d->meta + (size_t)row0 * (size_t)G * 4u;
  const uint32_t tbytes = (uint32_t)nrows * row_bytes, tmbytes = (uint32_t)nrows * (uint32_t)G * 4u;
  const uint32_t vco = (uint32_t)unit * (uint32_t)R * row_bytes + (uint32_t)q * 64u + (uint32_t)sub * 16u;
  const uint32_t vmo = (uint32_t)(unit * RG + ul) * 4u;
  uint32_t ico = 0, imo = 0;
  const uint32_t iend = (uint32_t)passes * 128u, mend = (uint32_t)((passes + 3) >> 2) * 32u;
  u32x4 cb[kInt4Depth];
  uint32_t mw[2];
  auto issue = [&](int slot) {  // the next pass's codes
    __builtin_amdgcn_s_setprio(1);
    const uint32_t n = ico < iend ? (uint32_t)max((int)tbytes - (int)ico, 0) : 0u;
    cb[slot] = load16_nt(make_rsrc(tcodes + ico, n), vco);
    __builtin_amdgcn_s_setprio(0);
    ico += 128u;
  };
  auto issue_meta = [&](int slot) {  // the next metadata block
    const uint32_t nm = imo < mend ? (uint32_t)max((int)tmbytes - (int)imo, 0) : 0u;
    mw[slot] = load4(make_rsrc(tmeta + imo, nm), vmo);
    imo += 32u;
  };
  issue_meta(0);
  issue_meta(1);
#pragma unroll
  for (int k = 0; k < kInt4Depth; ++k) issue(k);

  // LDS staging: x in the unpack order (chunk c's pairs (x0, x4), (x1, x5),
  // (x2, x6), (x3, x7) of each 8-element word) and zeroed row slots.
  {
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(d->x, (uint32_t)K * 2u);
    const int C = K >> 5;
    for (int i = threadIdx.x; i < xper * 4; i += 64 * kWaves) {
      const int c = i < C ? i : i - C;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x4 v = load16(xr, (uint32_t)c * 64u + 16u * w);
        u32x4 pz;
        pz[0] = __builtin_amdgcn_perm(v[2], v[0], 0x05040100u);
        pz[1] = __builtin_amdgcn_perm(v[2], v[0], 0x07060302u);
        pz[2] = __builtin_amdgcn_perm(v[3], v[1], 0x05040100u);
        pz[3] = __builtin_amdgcn_perm(v[3], v[1], 0x07060302u);
        *reinterpret_cast<u32x4*>(&xl[16 * i + 4 * w]) = pz;
      }
    }
    for (int i = threadIdx.x; i < 8 * rpt; i += 64 * kWaves) pl[i] = 0.0f;
  }
  __syncthreads();

  const uint32_t m0 = in_sgpr(0x000F000Fu), m1 = in_sgpr(0x00F000F0u);
  const uint32_t g1024 = in_vgpr(kMagic), g64 = in_vgpr(kMagic64);
  const char* xlane = (const char*)xl + q * 256 + sub * 64;  // plus (2 p mod xper) * 256
  char* plane = reinterpret_cast<char*>(pl + 8 * unit * R + ul);  // row r's slot: + 32 r bytes
  const uint32_t q32 = (uint32_t)q * 32u;
  const uint64_t kQuad0 = 0x5555555555555555ull;        // lanes of quad 0 in every unit
  // Pass state (wave-uniform): group index within the row of quad 0's group
  // (c0) and its row within the unit (as roff); x offset of the pass.
  int c0 = 0;
  uint32_t roff = 0;  // 32 r0: byte offset of row r0's slots
  uint32_t xo = 0;
  const uint32_t xwrap = (uint32_t)xper * 256u;
  float acc = 0.0f;
  for (int b = 0; b < passes; b += kInt4Unroll) {
#pragma unroll
    for (int k = 0; k < kInt4Unroll; ++k) {
      const int p = b + k;
      if (p < passes) {
        const u32x4* xp = reinterpret_cast<const u32x4*>(xlane + xo);
        const u32x4 xv[4] = {xp[0], xp[1], xp[2], xp[3]};
        uint32_t m;
        switch (k & 3) {
          case 0: m = quad_meta<0>(mw[k >> 2]); break;
          case 1: m = quad_meta<1>(mw[k >> 2]); break;
          case 2: m = quad_meta<2>(mw[k >> 2]); break;
          default: m = quad_meta<3>(mw[k >> 2]); break;
        }
        const h2 zz = bcast_hi(m);
        const h2 c1 = zz + as_h2(g1024), c64 = zz + as_h2(g64);
        float dv = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t v = cb[k % kInt4Depth][w], t = v >> 8;
          dv = __builtin_amdgcn_fdot2(as_h2((v & m0) | g1024) - c1, as_h2(xv[w][0]), dv, false);
          dv = __builtin_amdgcn_fdot2(as_h2((v & m1) | g64) - c64, as_h2(xv[w][1]), dv, false);
          dv = __builtin_amdgcn_fdot2(as_h2((t & m0) | g1024) - c1, as_h2(xv[w][2]), dv, false);
          dv = __builtin_amdgcn_fdot2(as_h2((t & m1) | g64) - c64, as_h2(xv[w][3]), dv, false);
        }
        const float a = fmaf(half_lo(m), dv, acc);
        // Quad 1's group of this pass: c0 + 1 within row r0, or the next row.
        const bool wrap = c0 + 1 == G;
        const int c1g = wrap ? 0 : c0 + 1;
        const bool last_odd = odd && p == passes - 1;    // quad 1 has no group
        if (last_odd) acc = __builtin_amdgcn_inverse_ballot_w64(kQuad0) ? a : acc;
        else acc = a;
        // quads whose row ends with this pass
        const uint64_t fm = (c0 + 2 >= G ? kQuad0 : 0ull) | (c1g + 2 >= G && !last_odd ? ~kQuad0 : 0ull);
        if (fm) {
          if (__builtin_amdgcn_inverse_ballot_w64(fm)) {
            *reinterpret_cast<float*>(plane + roff + (wrap ? q32 : 0u)) = acc;
            acc = 0.0f;
          }
        }
        c0 += 2;
        if (c0 >= G) { c0 -= G; roff += 32u; }
        if (c0 >= G) { c0 -= G; roff += 32u; }
        xo += 512u;
        if (xo >= xwrap) xo -= xwrap;
      }
      issue(k % kInt4Depth);
      if ((k & 3) == 3) issue_meta(k >> 2);  // after the block's last pass has read it
    }
  }
  __syncthreads();

  // Rows of the tile: the sum of their eight slots (pairwise, fixed order).
  const __amdgpu_buffer_rsrc_t yr = make_rsrc((char*)d->y + (size_t)row0 * 2u, (uint32_t)nrows * 2u);
  uint64_t best = 0;
  for (int r = threadIdx.x; r < nrows; r += 64 * kWaves) {
    const float4 u = reinterpret_cast<const float4*>(pl)[2 * r], v = reinterpret_cast<const float4*>(pl)[2 * r + 1];
    const uint16_t h = half_bits(((u.x + u.y) + (u.z + u.w)) + ((v.x + v.y) + (v.z + v.w)));
    store2(yr, (uint32_t)r * 2u, h);
    if (GREEDY && track) best = max_u64(best, greedy_key_f16(h, (uint32_t)(row0 + r)));
  }

  if constexpr (GREEDY) {
    if (track) {  // uniform over the workgroup
      best = wave_max_u64(best);
      const int wave = threadIdx.x >> 6;
      if (lane == 0) wave_best[wave] = best;
      __syncthreads();
      if (threadIdx.x == 0) {
        uint64_t bb = wave_best[0];
        for (int w = 1; w < kWaves; ++w) bb = max_u64(bb, wave_best[w]);
        g.slots[tile - d->work0] = bb;
      }
    }
  }
}

// One workgroup: the largest key over the target's tile slots -> its row.
__global__ __launch_bounds__(256) void greedy_finish_kernel(const tkq_gemv_desc* __restrict__ descs, int count,
                                                            int target, int tiles,
                                                            const uint64_t* __restrict__ slots,
                                                            int32_t* __restrict__ token) {
  __shared__ unsigned long long wave_best[kWaves];
  const int first = descs[target].work0;
  const int n = (target + 1 < count ? descs[target + 1].work0 : tiles) - first;
  uint64_t best = 0;
  for (int i = threadIdx.x; i < n; i += 64 * kWaves) best = max_u64(best, slots[i]);
  best = wave_max_u64(best);
  if ((threadIdx.x & 63) == 0) wave_best[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t b = wave_best[0];
    for (int w = 1; w < kWaves; ++w) b = max_u64(b, wave_best[w]);
    *token = (int32_t)(0xFFFFFFFFu - (uint32_t)b);
  }
}

template <int FMT>
constexpr int max_passes() {
  return FMT == kFmtBin ? 8 : ((FMT == kFmtTern || FMT == kFmtInt2) ? 3 : (FMT == kFmtInt3 ? 2 : 4));
}

typedef void (*GemvFn)(const tkq_gemv_desc*, int, Greedy);

template <int FMT, bool GREEDY>
GemvFn pick_variant(int jmax) {
  switch (jmax) {
    case 1: return gemv_kernel<FMT, 1, GREEDY>;
    case 2: return gemv_kernel<FMT, 2, GREEDY>;
    case 3: return gemv_kernel<FMT, 3, GREEDY>;
    case 4: return gemv_kernel<FMT, 4, GREEDY>;
  }
  if constexpr (max_passes<FMT>() > 4) return gemv_kernel<FMT, max_passes<FMT>(), GREEDY>;
  return nullptr;
}

template <int FMT>
GemvFn pick(int jmax, bool greedy) {
  return greedy ? pick_variant<FMT, true>(jmax) : pick_variant<FMT, false>(jmax);
}

}  // namespace

int gemv_max_passes(int fmt) {
  switch (fmt) {
    case kFmtInt4: return max_passes<kFmtInt4>();
    case kFmtHier: return max_passes<kFmtHier>();
    case kFmtInt2: return max_passes<kFmtInt2>();
    case kFmtInt3: return max_passes<kFmtInt3>();
    case kFmtK5: return max_passes<kFmtK5>();
    case kFmtTern: return max_passes<kFmtTern>();
    case kFmtBin: return max_passes<kFmtBin>();
  }
  return 0;
}

hipError_t launch_gemv(int fmt, int jmax, const tkq_gemv_desc* dev_descs, int count, int64_t tiles,
                       int target, int32_t* token, uint64_t* slots, hipStream_t stream) {
  const bool greedy = target >= 0;
  GemvFn fn = nullptr;
  size_t lds = 0;
  switch (fmt) {
    case kFmtInt4:  // jmax: the launch's dynamic LDS bytes
      if (jmax < 1 || jmax > kInt4MaxLds) return hipErrorInvalidValue;
      fn = greedy ? gemv_int4_kernel<true> : gemv_int4_kernel<false>;
      lds = (size_t)jmax;
      if (lds > 64 * 1024) {  // above the default dynamic-LDS limit (once per kernel; idempotent)
        static bool raised[2] = {false, false};
        if (!raised[greedy]) {
          const hipError_t e =
              hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, kInt4MaxLds);
          if (e != hipSuccess) return e;
          raised[greedy] = true;
        }
      }
      break;
    case kFmtHier: fn = pick<kFmtHier>(jmax, greedy); break;
    case kFmtInt2: fn = pick<kFmtInt2>(jmax, greedy); break;
    case kFmtInt3: fn = pick<kFmtInt3>(jmax, greedy); break;
    case kFmtK5: fn = pick<kFmtK5>(jmax, greedy); break;
    case kFmtTern: fn = pick<kFmtTern>(jmax, greedy); break;
    case kFmtBin: fn = pick<kFmtBin>(jmax, greedy); break;
  }
  if (!fn) return hipErrorInvalidValue;
  const Greedy g = {target, slots};
  hipLaunchKernelGGL(fn, dim3((uint32_t)tiles), dim3(64 * kWaves), lds, stream, dev_descs, count, g);
  if (greedy && token) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(greedy_finish_kernel, dim3(1), dim3(64 * kWaves), 0, stream, dev_descs, count, target,
                       (int)tiles, (const uint64_t*)slots, token);
  }
  return hipGetLastError();
}

}  // namespace tkq

// Prefill GEMM over int4 g128 weights for gfx950: Y = X . dequant(W)^T.
//
// With M >= 64 tokens per weight the product is a dense contraction (the
// Whetstone README, "Prior art": fast low-bit arithmetic helps only where many
// tokens share each weight, i.e. prefill and speculative verification, which
// are compute-bound), so this is the one place the library uses the matrix
// cores.  As in TKintegers K5 ("What is K5?"), low-bit codes are expanded to
// fp16 operands and multiplied with fp32 accumulation:
//
//  * A workgroup (4 wave64s) owns a BM x 256 tile of Y; wave w owns its 64
//    weight rows (columns of Y) and all BM tokens, so every weight is
//    dequantized by exactly one wave of the tile and needs no LDS.  Each
//    lane loads 16 bytes of codes per K step and 32-row block straight from
//    HBM and unpacks them in registers into a v_mfma_f32_32x32x16_f16
//    operand: the low nibbles of a word under the fp16 magic 1024.0 and its
//    next-to-low nibbles under 64.0 give (q0,q4), (q1,q5), (q2,q6), (q3,q7)
//    exactly; subtracting (magic + z) is exact and the product with the
//    fp16 scale rounds once.  The weight operand therefore holds k offsets
//    0,4,1,5,2,6,3,7 of each 8-block, and the activations are stored in LDS
//    in that order, so both operands agree on k.  The weights are the MFMA's
//    A operand, so each lane ends with four adjacent outputs of one token
//    per register quad (8- or 16-byte stores).
//  * The activations (shared by the 4 waves) are staged through LDS, two
//    stages, one barrier per K step of 64 (half a quantization group: one
//    (scale, zero) per weight row per step).  Codes are requested four K
//    steps ahead; a step's MFMAs run while the next step's codes are
//    unpacked (two register sets of weight operands).
//  * Split-K (optional, caller workspace): a work item may cover a K range
//    only; its fp32 partial tile goes to the workspace and a second kernel
//    sums the partials in a fixed order.  Without split-K the fp32
//    accumulators are rounded to fp16 (nearest even) on store.
#include "device_common.h"
#include "kernels.h"

namespace tkq {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;        // K step: half a quantization group
constexpr int WN = 64;        // weight rows per wave (two 32-row MFMA blocks)
constexpr int BN = 4 * WN;    // weight rows per workgroup tile
constexpr int DC = 4;         // code ring slots (K steps in flight)
constexpr int kXcds = 8;      // accelerator complexes of the part (L2 domains)
constexpr int LDSW = BK + 8;  // halfs per LDS row of activations (16 bytes of padding)
constexpr uint32_t kMagicLo = 0x64006400u;  // fp16 pair (1024, 1024): ulp 1
constexpr uint32_t kMagicHi = 0x54005400u;  // fp16 pair (64, 64): ulp 1/16
constexpr uint32_t kDead = 0x80000000u;     // buffer offset past every range: loads return 0

template <int N>
struct Slot {
  static constexpr int value = N;
};

// Constants in registers: a gfx9 VOP3 instruction (v_and_or_b32) can encode
// no literal and read at most one SGPR, so the masks live in SGPRs and the
// magic numbers in VGPRs.
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

struct DqRegs {
  uint32_t mlo, mhi;  // 0x000F000F, 0x00F000F0
  uint32_t glo, ghi;  // the magic pairs
};
__device__ __forceinline__ DqRegs dq_regs() {
  return {in_sgpr(0x000F000Fu), in_sgpr(0x00F000F0u), in_vgpr(kMagicLo), in_vgpr(kMagicHi)};
}

// Per weight row and group: the subtrahends (1024 + z, 64 + z) and the scale
// as fp16 pairs.  z is an integer 0..15, so both sums are exact.
struct RowMeta {
  h2 zlo, zhi, s;
};
__device__ __forceinline__ RowMeta row_meta(uint32_t m) {
  const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(m & 0xFFFFu));
  const _Float16 z = __builtin_bit_cast(_Float16, (uint16_t)(m >> 16));
  const _Float16 lo = (_Float16)1024.0f + z, hi = (_Float16)64.0f + z;
  return {h2{lo, lo}, h2{hi, hi}, h2{s, s}};
}

// Code word v (nibble i = weight k0 + i) -> the 8 fp16 weights s*(q - z) in
// the order k0 + {0,4,1,5,2,6,3,7}.
__device__ __forceinline__ half8 dq_word(uint32_t v, const RowMeta& r, const DqRegs& R) {
  const uint32_t v8 = v >> 8;
  const h2 p0 = (as_h2((v & R.mlo) | R.glo) - r.zlo) * r.s;    // (q0, q4)
  const h2 p1 = (as_h2((v & R.mhi) | R.ghi) - r.zhi) * r.s;    // (q1, q5)
  const h2 p2 = (as_h2((v8 & R.mlo) | R.glo) - r.zlo) * r.s;   // (q2, q6)
  const h2 p3 = (as_h2((v8 & R.mhi) | R.ghi) - r.zhi) * r.s;   // (q3, q7)
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 8 activations x[k0..k0+7] (one 16-byte load) -> the order k0 + {0,4,1,5,2,6,3,7}.
__device__ __forceinline__ u32x4 perm_x(u32x4 d) {
  return u32x4{__builtin_amdgcn_perm(d[2], d[0], 0x05040100u), __builtin_amdgcn_perm(d[2], d[0], 0x07060302u),
               __builtin_amdgcn_perm(d[3], d[1], 0x05040100u), __builtin_amdgcn_perm(d[3], d[1], 0x07060302u)};
}

// splits > 1: partial fp32 tiles into part[z][M][N]; else fp16 Y.
template <int MB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MB >= 8 ? 1 : 2, MB >= 8 ? 1 : 2))) void
prefill_kernel(const uint16_t* __restrict__ X, const uint32_t* __restrict__ codes, const uint32_t* __restrict__ meta,
               uint16_t* __restrict__ Y, float* __restrict__ part, int M, int N, int K, int ksteps_per_split,
               int tsplit, int full_x) {
  constexpr int BM = 32 * MB;
  constexpr int XV = BM * BK * 2 / 16 / 256;  // 16-byte activation loads per thread and K step
  __shared__ __attribute__((aligned(16))) _Float16 xs[2][BM * LDSW];

  // Work item -> (split, N tile, M tile), M fastest: the M tiles that share
  // one weight tile are consecutive.  Workgroup b runs on XCD b % 8, and the
  // work items of one XCD are a contiguous range, so those M tiles also
  // share that XCD's L2.
  const int MT = (M + BM - 1) / BM;
  const int total = (int)gridDim.x;
  const int xcd = (int)blockIdx.x % kXcds;
  int split, tile;
  if (tsplit > 1) {
    // Tail split: in each XCD's range, the tiles of its last, partial round
    // are cut into tsplit K pieces (fp32 partials, summed by
    // tail_reduce_kernel), so that round fills the XCD's slots.
    // full_x: tiles of the full rounds (the same for every XCD); the XCD's
    // remaining tiles (at most one round) are the split ones.
    const int k = (int)blockIdx.x / kXcds;
    const int T = MT * ((N + BN - 1) / BN), per = T / kXcds, rem = T % kXcds;
    const int tiles_x = per + (xcd < rem ? 1 : 0), start_x = xcd * per + min(xcd, rem);
    const int last = tiles_x - full_x;
    if (k < full_x) {
      tile = start_x + k;
      split = -1;
    } else {
      const int j = k - full_x;
      if (j >= last * tsplit) return;  // padding of the grid (uniform: the whole workgroup leaves)
      tile = start_x + full_x + j / tsplit;
      split = j % tsplit;
    }
  } else {
    const int per = total / kXcds, rem = total % kXcds;
    const int work = xcd * per + min(xcd, rem) + (int)blockIdx.x / kXcds;
    const int T = MT * ((N + BN - 1) / BN);
    split = work / T;
    tile = work - split * T;
  }
  const int m0 = (tile % MT) * BM, n0 = (tile / MT) * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mrows = min(BM, M - m0);
  const int w0 = n0 + wave * WN, wrows = max(0, min(WN, N - w0));  // this wave's weight rows
  const int kbeg = split > 0 ? split * ksteps_per_split * BK : 0;
  const int kend = split < 0 ? K : min(K, kbeg + ksteps_per_split * BK);  // split < 0: a whole tile
  const int nk = (kend - kbeg) / BK;
  const uint32_t xrow = (uint32_t)K * 2u, crow = (uint32_t)K / 2u, mrow = (uint32_t)(K / 128) * 4u;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X + (size_t)m0 * K, (uint32_t)mrows * xrow);
  const __amdgpu_buffer_rsrc_t cr =
      make_rsrc_uniform((const char*)codes + (size_t)max(w0, 0) * crow, 0u, (uint32_t)wrows * crow);
  const __amdgpu_buffer_rsrc_t mr =
      make_rsrc_uniform((const char*)meta + (size_t)max(w0, 0) * mrow, 0u, (uint32_t)wrows * mrow);

  // Lane l: weight row 32 b + l % 32 of the wave (b = MFMA block), k half
  // l / 32 of a K step (its 16-byte chunk = 32 weights = 4 code words).
  const int half = lane >> 5, lrow = lane & 31;
  uint32_t coff[2], moff[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    coff[b] = (uint32_t)(b * 32 + lrow) * crow + (uint32_t)half * 16u;
    moff[b] = (uint32_t)(b * 32 + lrow) * mrow;
  }
  // Step t's offset within a row, or an offset past every range for steps
  // beyond this work item's K range (their loads return 0 and move no data);
  // wave-uniform, so the selection is scalar.
  auto kofs = [&](int t) -> uint32_t { return t < nk ? (uint32_t)(kbeg + t * BK) : kDead; };
  // kDead / 2 and kDead / 32 still lie past every code and metadata range
  auto code_off = [&](int b, int t) -> uint32_t { return coff[b] + (kofs(t) >> 1); };
  auto meta_off = [&](int b, int t) -> uint32_t { return moff[b] + ((kofs(t) >> 7) << 2); };
  auto x_off = [&](int i, int t) -> uint32_t {
    const int idx = i * 256 + tid, r = idx >> 3, c = idx & 7;  // 8 x 16 B per 64-half row
    return (uint32_t)r * xrow + (uint32_t)c * 16u + (t < nk ? (uint32_t)(kbeg + t * BK) * 2u : kDead);
  };
  auto x_store = [&](const u32x4* xv, int t) {
    _Float16* dst = xs[t & 1];
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int idx = i * 256 + tid, r = idx >> 3, c = idx & 7;
      *reinterpret_cast<u32x4*>(&dst[r * LDSW + c * 8]) = perm_x(xv[i]);
    }
  };

  f32x16 acc[MB][2];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  const DqRegs dqr = dq_regs();
  u32x4 xv[XV];
  u32x4 cw[DC][2];
  uint32_t mw[DC][2];
  half8 bf[2][2][4];  // B operands of two K steps: [step parity][MFMA block][word]
  auto load_codes = [&](int s, int t) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      cw[s][b] = load16(cr, code_off(b, t));
      mw[s][b] = load4(mr, meta_off(b, t));
    }
  };
  auto unpack = [&](int s, int p) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const RowMeta rm = row_meta(mw[s][b]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[p][b][j] = dq_word(cw[s][b][j], rm, dqr);
    }
  };
  // Prologue: activations of step 0 (waited for below), codes of steps
  // 0..DC-1, activations of step 1; step 0's codes unpacked and their slot
  // refilled with step DC.
#pragma unroll
  for (int i = 0; i < XV; ++i) xv[i] = load16(xr, x_off(i, 0));
#pragma unroll
  for (int s = 0; s < DC; ++s) load_codes(s, s);
  x_store(xv, 0);
#pragma unroll
  for (int i = 0; i < XV; ++i) xv[i] = load16(xr, x_off(i, 1));
  unpack(0, 0);
  load_codes(0, DC);
  __syncthreads();

  // One K step t (I = t % DC): the MFMAs of step t on B operands bf[I % 2],
  // interleaved with unpacking step t+1 (code slot (I+1) % DC) into
  // bf[(I+1) % 2] and refilling that slot with step t+1+DC.
  constexpr int NMF = MB * 8;                  // MFMAs per step
  constexpr int NVALU = (120 + NMF - 1) / NMF;  // unpack VALU slots per MFMA
  auto step = [&](auto slot, int t) {
    constexpr int I = decltype(slot)::value;
    constexpr int P = I % 2, S1 = (I + 1) % DC;
    // activations of step t+1 into the other LDS stage (free since the last
    // barrier), then request those of step t+2 (before this step's code
    // loads, so that waiting for them never waits for codes)
    x_store(xv, t + 1);
#pragma unroll
    for (int i = 0; i < XV; ++i) xv[i] = load16(xr, x_off(i, t + 2));
    __builtin_amdgcn_sched_barrier(0);
    unpack(S1, P ^ 1);
    load_codes(S1, t + 1 + DC);
    const _Float16* xb = xs[t & 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8 fa[MB];
#pragma unroll
      for (int a = 0; a < MB; ++a)
        fa[a] = *reinterpret_cast<const half8*>(&xb[(a * 32 + lrow) * LDSW + half * 32 + j * 8]);
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[P][b][j], fa[a], acc[a][b], 0, 0, 0);
    }
    // Issue order: the first sub-step's A operands, then each MFMA followed
    // by unpack work; the next sub-step's A operands spread over the MFMAs
    // of the current one, the code loads in the middle.
    __builtin_amdgcn_sched_group_barrier(0x100, MB, 0);
#pragma unroll
    for (int k = 0; k < NMF; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);
      if (k % 2 == 1 && k < NMF - 2 * MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (k == NMF / 2) __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
    }
    __syncthreads();
  };

  int t = 0;
  for (; t + DC <= nk; t += DC) {
    step(Slot<0>{}, t);
    step(Slot<1>{}, t + 1);
    step(Slot<2>{}, t + 2);
    step(Slot<3>{}, t + 3);
  }
  if (t < nk) step(Slot<0>{}, t);
  if (t + 1 < nk) step(Slot<1>{}, t + 1);
  if (t + 2 < nk) step(Slot<2>{}, t + 2);

  // D layout of a 32x32 fp32 accumulator (weights as the A operand): register
  // r of lane l holds weight row 8*(r/4) + 4*(l/32) + r%4 of the block and
  // token l%32, so registers 4q..4q+3 are four adjacent outputs of one token:
  // one 8-byte (fp16) or 16-byte (fp32 partial) store when N % 4 == 0.
  float* pz = (part && split >= 0) ? part + (size_t)split * M * N : nullptr;
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int a = 0; a < MB; ++a) {
    const int m = a * 32 + lrow;
    if (m >= mrows) continue;
    const size_t orow = (size_t)(m0 + m) * N + w0;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = b * 32 + 8 * q + 4 * half;
        const float v[4] = {acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]};
        if (vec && n + 3 < wrows) {
          if (pz) {
            *reinterpret_cast<float4*>(pz + orow + n) = float4{v[0], v[1], v[2], v[3]};
          } else {
            const uint32_t lo = half_bits(v[0]) | ((uint32_t)half_bits(v[1]) << 16);
            const uint32_t hi = half_bits(v[2]) | ((uint32_t)half_bits(v[3]) << 16);
            *reinterpret_cast<uint2*>(Y + orow + n) = uint2{lo, hi};
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < wrows) {
              if (pz) pz[orow + n + e] = v[e];
              else Y[orow + n + e] = half_bits(v[e]);
            }
        }
      }
  }
}

// Y = fp16(sum over z of part[z]), summed in z order; four elements per
// thread step where MN % 4 == 0.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            uint16_t* __restrict__ Y, int64_t MN, int splits) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  if ((MN & 3) == 0) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < MN / 4; i += stride) {
      float4 v = reinterpret_cast<const float4*>(part)[i];
      for (int z = 1; z < splits; ++z) {
        const float4 w = reinterpret_cast<const float4*>(part + (size_t)z * MN)[i];
        v.x += w.x;
        v.y += w.y;
        v.z += w.z;
        v.w += w.w;
      }
      reinterpret_cast<uint2*>(Y)[i] = uint2{half_bits(v.x) | ((uint32_t)half_bits(v.y) << 16),
                                             half_bits(v.z) | ((uint32_t)half_bits(v.w) << 16)};
    }
    return;
  }
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < MN; i += stride) {
    float v = part[i];
    for (int z = 1; z < splits; ++z) v += part[(size_t)z * MN + i];
    Y[i] = half_bits(v);
  }
}

// Y of the tail tiles = fp16(sum over the tsplit partials), in piece order.
// Grid: (XCD, tail tile of that XCD, element chunks); four adjacent outputs
// per thread step.
__global__ __launch_bounds__(256) void tail_reduce_kernel(const float* __restrict__ part, uint16_t* __restrict__ Y,
                                                          int M, int N, int BM, int BN, int tsplit, int full_x) {
  const int MT = (M + BM - 1) / BM, NT = (N + BN - 1) / BN, T = MT * NT;
  const int xcd = blockIdx.x, i = blockIdx.y;
  const int per = T / kXcds, rem = T % kXcds;
  const int tiles_x = per + (xcd < rem ? 1 : 0), start_x = xcd * per + min(xcd, rem);
  if (i >= tiles_x - full_x) return;
  const int tile = start_x + full_x + i;
  const int m0 = (tile % MT) * BM, n0 = (tile / MT) * BN;
  const size_t MN = (size_t)M * N;
  const bool vec = (N & 3) == 0;
  for (int e = (blockIdx.z * 256 + threadIdx.x) * 4; e < BM * BN; e += 1024 * gridDim.z) {
    const int r = e / BN, c = e - r * BN;
    if (m0 + r >= M) continue;
    const size_t o = (size_t)(m0 + r) * N + n0 + c;
    if (vec && n0 + c + 3 < N) {
      float4 v = *reinterpret_cast<const float4*>(part + o);
      for (int z = 1; z < tsplit; ++z) {
        const float4 w = *reinterpret_cast<const float4*>(part + (size_t)z * MN + o);
        v.x += w.x;
        v.y += w.y;
        v.z += w.z;
        v.w += w.w;
      }
      *reinterpret_cast<uint2*>(Y + o) = uint2{half_bits(v.x) | ((uint32_t)half_bits(v.y) << 16),
                                               half_bits(v.z) | ((uint32_t)half_bits(v.w) << 16)};
    } else {
      for (int u = 0; u < 4; ++u) {
        if (n0 + c + u >= N) break;
        float v = part[o + u];
        for (int z = 1; z < tsplit; ++z) v += part[(size_t)z * MN + o + u];
        Y[o + u] = half_bits(v);
      }
    }
  }
}

struct Config {
  int mb, splits;      // tile BM = 32 * mb rows by BN; K split over `splits` work items
  int tsplit, full_x;  // tail split (1: none); tiles per XCD in its full rounds
};

// Resident workgroups per CU of each tile height (registers: MB = 8 holds
// 256 fp32 accumulators per lane, one wave per SIMD; MB = 2 runs at two).
constexpr int per_cu(int mb) { return mb >= 8 ? 1 : 2; }

// Pick the tile height that keeps the most of the GPU's workgroup slots busy
// over whole rounds, weighted by its unpack work per MFMA (every M tile
// unpacks its weight tile again; MB = 2 is bound by that vector work) and by
// the share of its tile rows that hold tokens (so short M takes MB = 2).  With
// a workspace, a shape that leaves slots idle may split K: the smallest split
// that fills 80 % of the slots.  A shape with more than one round may
// instead split the tiles of its last, partial round (tail split).
Config choose(int64_t M, int64_t N, int64_t K, int cus, int64_t ws_floats) {
  struct Cand {
    int mb;
    double eff;
  };
  const Cand cands[] = {{8, 1.0}, {2, 0.6}};
  const int64_t ksteps = (K + BK - 1) / BK;
  auto split_for = [&](int64_t tiles, int64_t slots) {
    int s = 1;
    if (tiles < slots) {
      for (int t = 2; t <= 8; ++t) {
        if ((int64_t)t * M * N > ws_floats || t > ksteps / 4) break;
        s = t;
        if (tiles * t * 5 >= slots * 4) break;
      }
    }
    return s;
  };
  Config best = {4, 1, 1, 0};
  double best_score = -1.0;
  for (const Cand& c : cands) {
    const int bm = 32 * c.mb;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + BN - 1) / BN);
    const int64_t slots = (int64_t)cus * per_cu(c.mb);
    const int64_t items = tiles * split_for(tiles, slots);
    const int64_t rounds = (items + slots - 1) / slots;
    // rows of the M tiles that hold tokens (M = 64 in 256-row tiles wastes 3/4 of the MFMAs)
    const double fill = double(M) / double(((M + bm - 1) / bm) * bm);
    const double score = double(items) / double(rounds * slots) * c.eff * fill;
    if (score > best_score + 1e-9) {
      best_score = score;
      best = {c.mb, 1, 1, 0};
    }
  }
  const int bm = 32 * best.mb;
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + BN - 1) / BN);
  const int64_t slots = (int64_t)cus * per_cu(best.mb);
  if (tiles < slots) {
    best.splits = split_for(tiles, slots);
  } else if (cus % kXcds == 0) {
    // Tail split: the rounds are those of the largest XCD range; every XCD
    // cuts the tiles after its full rounds (at most `last`) into s pieces,
    // the largest s with s * last within one round of slots.
    const int64_t sx = slots / kXcds, tiles_x = tiles / kXcds + (tiles % kXcds ? 1 : 0);
    const int64_t rounds = (tiles_x + sx - 1) / sx;
    const int64_t last = tiles_x - (rounds - 1) * sx;
    for (int s = 4; s >= 2; --s) {
      if (last * s <= sx && (int64_t)s * M * N <= ws_floats && s <= ksteps / 4) {
        best.tsplit = s;
        best.full_x = (int)((rounds - 1) * sx);
        break;
      }
    }
  }
  return best;
}

template <int MB>
void launch_tile(int64_t M, int64_t N, int64_t K, const Config& c, const uint32_t* codes, const uint32_t* meta,
                 const uint16_t* X, uint16_t* Y, float* part, hipStream_t stream) {
  constexpr int BM = 32 * MB;
  const int64_t ksteps = (K + BK - 1) / BK;
  const int64_t T = ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
  if (c.tsplit > 1) {
    // per XCD: the full-round tiles, then tsplit pieces of each remaining
    // tile; grid = 8 x the largest XCD's item count
    const int64_t tiles_x = T / kXcds + (T % kXcds ? 1 : 0);
    const int64_t items = c.full_x + (tiles_x - c.full_x) * c.tsplit;
    const int per_piece = (int)((ksteps + c.tsplit - 1) / c.tsplit);
    hipLaunchKernelGGL((prefill_kernel<MB>), dim3((uint32_t)(items * kXcds)), dim3(256), 0, stream, X, codes, meta,
                       Y, part, (int)M, (int)N, (int)K, per_piece, c.tsplit, c.full_x);
    return;
  }
  const int per_split = (int)((ksteps + c.splits - 1) / c.splits);
  hipLaunchKernelGGL((prefill_kernel<MB>), dim3((uint32_t)(T * c.splits)), dim3(256), 0, stream, X, codes, meta, Y,
                     part, (int)M, (int)N, (int)K, per_split, 1, 0);
}

}  // namespace

hipError_t launch_prefill(int64_t M, int64_t N, int64_t K, const uint32_t* codes, const uint32_t* meta,
                          const uint16_t* X, uint16_t* Y, float* workspace, int64_t workspace_bytes,
                          hipStream_t stream) {
  int device = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &device) : hipGetDevice(&device);
  if (e != hipSuccess) return e;
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return e;
  const Config c = choose(M, N, K, cus > 0 ? cus : 1, workspace ? workspace_bytes / 4 : 0);
  float* part = (c.splits > 1 || c.tsplit > 1) ? workspace : nullptr;
  if (c.mb == 8) launch_tile<8>(M, N, K, c, codes, meta, X, Y, part, stream);
  else launch_tile<2>(M, N, K, c, codes, meta, X, Y, part, stream);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (c.tsplit > 1) {
    const int bm = 32 * c.mb;
    const int64_t T = ((N + BN - 1) / BN) * ((M + bm - 1) / bm);
    const int64_t last = T / kXcds + (T % kXcds ? 1 : 0) - c.full_x;
    hipLaunchKernelGGL(tail_reduce_kernel, dim3(kXcds, (uint32_t)last, 16), dim3(256), 0, stream, workspace, Y,
                       (int)M, (int)N, bm, BN, c.tsplit, c.full_x);
    return hipGetLastError();
  }
  if (c.splits == 1) return e;
  const int64_t MN = M * N;
  int64_t blocks = ((MN % 4 ? MN : MN / 4) + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, workspace, Y, MN,
                     c.splits);
  return hipGetLastError();
}

}  // namespace tkq

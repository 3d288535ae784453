// Prefill GEMM over int4 g128 weights for gfx950: Y = X . dequant(W)^T.
//
// With M >= 64 tokens per weight the product is a dense contraction (the
// Whetstone README, "Prior art": fast low-bit arithmetic helps only where many
// tokens share each weight, i.e. prefill and speculative verification, which
// are compute-bound), so this is the one place the library uses the matrix
// cores.  As in
// TKintegers K5 ("What is K5?"), tiles of low-bit codes are expanded to fp16
// operands and multiplied with fp32 accumulation:
//
//  * A workgroup (4 wave64s, 2 x 2) owns a BM x BN tile of Y and walks its K
//    range in steps of 64 (half a quantization group, so each weight row of a
//    step has one (scale, zero) pair).
//  * Software pipeline: two LDS stages plus register rings.  While the MFMAs
//    consume step k from LDS, the global loads of later steps are in flight
//    in registers (weight codes + metadata DW steps ahead: they come from
//    HBM and cost 5 registers per step; activations DX steps ahead: they are
//    reused by every N tile and mostly hit L2).  Step k+1 is then written to
//    the other LDS stage (codes unpacked with the fp16 magic-number trick,
//    shifted by the zero point — exact small integers — and multiplied by the
//    fp16 scale: one fp16 rounding), and one barrier per step hands it over.
//  * Each wave computes a (BM/2) x (BN/2) sub-tile with
//    v_mfma_f32_32x32x16_f16 from 16-byte LDS reads; rows are padded by 16
//    bytes against bank conflicts.
//  * Split-K (optional, caller workspace): blockIdx.z selects a K range and
//    the fp32 partial tile goes to workspace[z]; a second kernel sums the
//    partials in a fixed order and rounds to fp16.  Without split-K the fp32
//    accumulators are rounded to fp16 (nearest even) on store.
#include "device_common.h"
#include "kernels.h"

namespace tkq {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int kXcds = 8;  // accelerator complexes of the part (L2 domains)
#ifndef TKQ_PREFILL_XCD
#define TKQ_PREFILL_XCD 1
#endif
constexpr int LDSW = BK + 8;  // halfs per LDS row (16 bytes of padding)
constexpr uint32_t kMagic = 0x64006400u;

// Constants held in registers: a gfx9 VOP3 instruction (v_perm_b32,
// v_and_or_b32) can encode no literal and read at most one SGPR, so the
// selectors and the mask live in SGPRs and the magic number in a VGPR.
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
  uint32_t sel[4];  // byte p of the code word -> bytes 0 and 2 of a pair word
  uint32_t mask;    // 0x000F000F
  uint32_t magic;   // fp16 pair (1024, 1024)
};
__device__ __forceinline__ DqRegs dq_regs() {
  return {{in_sgpr(0x0C040C00u), in_sgpr(0x0C050C01u), in_sgpr(0x0C060C02u), in_sgpr(0x0C070C03u)},
          in_sgpr(0x000F000Fu), in_vgpr(kMagic)};
}

// Code word v holds nibbles q0..q7 (q_{2p} in the low and q_{2p+1} in the
// high nibble of byte p).  Pair p: v_perm puts byte p of v and of v >> 4 into
// the two halves, v_and_or keeps their low nibbles under the fp16 magic
// 1024.0, giving (1024 + q_{2p}, 1024 + q_{2p+1}) exactly; subtracting
// (1024 + z) is exact and the product with the fp16 scale rounds once.
__device__ __forceinline__ uint32_t dq_pair(uint32_t v, uint32_t v4, uint32_t sel, const DqRegs& R, h2 zoff,
                                            h2 s) {
  const uint32_t u = __builtin_amdgcn_perm(v4, v, sel);
  const h2 h = as_h2((u & R.mask) | R.magic) - zoff;
  return __builtin_bit_cast(uint32_t, h * s);
}

// Global -> register staging of one K step, split in the X part (fp16
// activations, reused by every N tile, mostly served from L2) and the W part
// (int4 codes + metadata from HBM: 5 registers per stage, so it can be
// prefetched several steps ahead).
template <int BM>
struct XStage {
  static constexpr int XV = BM * BK * 2 / 16 / 256;  // 16-byte X loads per thread
  u32x4 x[XV];
};
template <int BN>
struct WStage {
  static constexpr int WV = BN * BK / 2 / 16 / 256;  // 16-byte code loads per thread (may be 0)
  static constexpr int WT = BN * BK / 2 / 16;        // code loads per step in total
  u32x4 w[WV > 0 ? WV : 1];
  uint32_t m[WV > 0 ? WV : 1];
};

template <int BM>
__device__ __forceinline__ void load_x(XStage<BM>& st, int k0, int tid, __amdgpu_buffer_rsrc_t xr, uint32_t xrow) {
#pragma unroll
  for (int i = 0; i < XStage<BM>::XV; ++i) {
    const int idx = i * 256 + tid, r = idx >> 3, c = idx & 7;  // 8 x 16 B per 64-half row
    st.x[i] = load16(xr, (uint32_t)r * xrow + (uint32_t)k0 * 2u + (uint32_t)c * 16u);
  }
}

template <int BN>
__device__ __forceinline__ void load_w(WStage<BN>& st, int k0, int tid, __amdgpu_buffer_rsrc_t cr,
                                       __amdgpu_buffer_rsrc_t mr, uint32_t crow, uint32_t mrow) {
  using S = WStage<BN>;
#pragma unroll
  for (int i = 0; i < (S::WV > 0 ? S::WV : 1); ++i) {
    const int idx = i * 256 + tid, r = idx >> 1, c = idx & 1;  // 2 x 16 B of codes per row
    const bool live = S::WV > 0 || idx < S::WT;
    st.w[i] = load16_nt(cr, live ? (uint32_t)r * crow + (uint32_t)k0 / 2u + (uint32_t)c * 16u : 0x80000000u);
    st.m[i] = load4(mr, live ? (uint32_t)r * mrow + (uint32_t)(k0 / 128) * 4u : 0x80000000u);
  }
}

template <int BM>
__device__ __forceinline__ void store_x(const XStage<BM>& st, _Float16* xs, int tid) {
#pragma unroll
  for (int i = 0; i < XStage<BM>::XV; ++i) {
    const int idx = i * 256 + tid, r = idx >> 3, c = idx & 7;
    *reinterpret_cast<u32x4*>(&xs[r * LDSW + c * 8]) = st.x[i];
  }
}

template <int BN>
__device__ __forceinline__ void store_w(const WStage<BN>& st, _Float16* ws, int tid, const DqRegs& R) {
  using S = WStage<BN>;
#pragma unroll
  for (int i = 0; i < (S::WV > 0 ? S::WV : 1); ++i) {
    const int idx = i * 256 + tid, r = idx >> 1, c = idx & 1;
    if (S::WV == 0 && idx >= S::WT) continue;
    const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(st.m[i] & 0xFFFFu));
    const _Float16 z = __builtin_bit_cast(_Float16, (uint16_t)(st.m[i] >> 16));
    const h2 ss = {s, s};
    const _Float16 zo = (_Float16)1024.0f + z;  // exact: z is an integer 0..15
    const h2 zoff = {zo, zo};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t v = st.w[i][w], v4 = v >> 4;
      u32x4 out;
#pragma unroll
      for (int p = 0; p < 4; ++p) out[p] = dq_pair(v, v4, R.sel[p], R, zoff, ss);  // (w_2p, w_2p+1)
      *reinterpret_cast<u32x4*>(&ws[r * LDSW + c * 32 + w * 8]) = out;
    }
  }
}

#ifndef TKQ_PREFILL_DW
#define TKQ_PREFILL_DW 1  // K steps of weight codes in flight
#endif
#ifndef TKQ_PREFILL_DX
#define TKQ_PREFILL_DX 1  // K steps of activations in flight
#endif
constexpr int DW = TKQ_PREFILL_DW, DX = TKQ_PREFILL_DX;
constexpr int UNR = DW > DX ? DW : DX;  // loop unroll: ring slots stay static
static_assert(UNR % DW == 0 && UNR % DX == 0, "ring sizes must divide the unroll");

// splits > 1: partial fp32 tiles into part[z][M][N]; else fp16 Y.
template <int BM, int BN>
__global__ __launch_bounds__(256) void prefill_kernel(const uint16_t* __restrict__ X,
                                                      const uint32_t* __restrict__ codes,
                                                      const uint32_t* __restrict__ meta,
                                                      uint16_t* __restrict__ Y, float* __restrict__ part,
                                                      int M, int N, int K, int ksteps_per_split, int tsplit,
                                                      int full_x) {
  constexpr int A = BM / 64, B = BN / 64;  // 32x32 MFMA tiles per wave in M and N
  static_assert(A >= 1 && B >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) _Float16 xs[2][BM * LDSW];
  __shared__ __attribute__((aligned(16))) _Float16 ws[2][BN * LDSW];

  // Work item -> (split, N tile, M tile), M fastest: the M tiles that share
  // one weight tile are consecutive.  With XCD-aware order the work items
  // of one XCD (workgroup b runs on XCD b % 8) are a contiguous range, so
  // those M tiles also share that XCD's L2.
  const int MT = (M + BM - 1) / BM, NT = (N + BN - 1) / BN;
  const int total = (int)gridDim.x;
#if TKQ_PREFILL_XCD
  const int xcd = (int)blockIdx.x % kXcds, per = total / kXcds, rem = total % kXcds;
  const int work = xcd * per + min(xcd, rem) + (int)blockIdx.x / kXcds;
#else
  const int work = (int)blockIdx.x;
#endif
  int split = work / (MT * NT), tile = work - split * (MT * NT);
  if (tsplit > 1) {
    // Tail split: in each XCD's range, the tiles of its last, partial round
    // are cut into tsplit K pieces (fp32 partials, summed by
    // tail_reduce_kernel), so that round fills the XCD's slots.
    // full_x: tiles of the full rounds (the same for every XCD); the XCD's
    // remaining tiles (at most one round) are the split ones.
    const int xcd = (int)blockIdx.x % kXcds, k = (int)blockIdx.x / kXcds;
    const int T = MT * NT, per = T / kXcds, rem = T % kXcds;
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
  }
  const int m0 = (tile % MT) * BM, n0 = (tile / MT) * BN;
  (void)NT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (BN / 2);
  const int mrows = min(BM, M - m0), nrows = min(BN, N - n0);
  const int kbeg = split > 0 ? split * ksteps_per_split * BK : 0;
  const int kend = split < 0 ? K : min(K, kbeg + ksteps_per_split * BK);  // split < 0: a whole tile
  const uint32_t xrow = (uint32_t)K * 2u, crow = (uint32_t)K / 2u, mrow = (uint32_t)(K / 128) * 4u;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X + (size_t)m0 * K, (uint32_t)mrows * xrow);
  const __amdgpu_buffer_rsrc_t cr = make_rsrc((const char*)codes + (size_t)n0 * crow, (uint32_t)nrows * crow);
  const __amdgpu_buffer_rsrc_t mr = make_rsrc((const char*)meta + (size_t)n0 * mrow, (uint32_t)nrows * mrow);

  f32x16 acc[A][B];
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // Prologue: weight steps 0..DW-1 and activation steps 0..DX-1 in flight,
  // step 0 staged to LDS.
  const int nk = (kend - kbeg) / BK;
  XStage<BM> xr_[DX];
  WStage<BN> wr_[DW];
#pragma unroll
  for (int i = 0; i < DW; ++i)
    if (i < nk) load_w<BN>(wr_[i], kbeg + i * BK, tid, cr, mr, crow, mrow);
#pragma unroll
  for (int i = 0; i < DX; ++i)
    if (i < nk) load_x<BM>(xr_[i], kbeg + i * BK, tid, xr, xrow);
  const DqRegs dqr = dq_regs();
  store_x<BM>(xr_[0], xs[0], tid);
  store_w<BN>(wr_[0], ws[0], tid, dqr);
  __syncthreads();

  for (int t0 = 0; t0 < nk; t0 += UNR) {
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      const int t = t0 + i;
      if (t < nk) {
        // refill the ring slots that step t used
        if (t + DX < nk) load_x<BM>(xr_[i % DX], kbeg + (t + DX) * BK, tid, xr, xrow);
        if (t + DW < nk) load_w<BN>(wr_[i % DW], kbeg + (t + DW) * BK, tid, cr, mr, crow, mrow);
        const _Float16* xb = xs[t & 1];
        const _Float16* wb = ws[t & 1];
#pragma unroll
        for (int ks = 0; ks < BK; ks += 16) {
          half8 fa[A], fb[B];
          const int kk = ks + (lane >> 5) * 8;
#pragma unroll
          for (int a = 0; a < A; ++a) fa[a] = *reinterpret_cast<const half8*>(&xb[(wm + a * 32 + (lane & 31)) * LDSW + kk]);
#pragma unroll
          for (int b = 0; b < B; ++b) fb[b] = *reinterpret_cast<const half8*>(&wb[(wn + b * 32 + (lane & 31)) * LDSW + kk]);
#pragma unroll
          for (int a = 0; a < A; ++a)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[a], fb[b], acc[a][b], 0, 0, 0);
        }
        if (t + 1 < nk) {  // stage step t+1 into the other LDS buffer
          store_x<BM>(xr_[(i + 1) % DX], xs[(t + 1) & 1], tid);
          store_w<BN>(wr_[(i + 1) % DW], ws[(t + 1) & 1], tid, dqr);
        }
        __syncthreads();
      }
    }
  }

  // D layout of a 32x32 fp32 accumulator: register r of lane l holds row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32.
  float* pz = (part && split >= 0) ? part + (size_t)split * M * N : nullptr;
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = wm + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int j = wn + b * 32 + (lane & 31);
        if (i < mrows && j < nrows) {
          const size_t o = (size_t)(m0 + i) * N + n0 + j;
          if (pz) pz[o] = acc[a][b][r];
          else Y[o] = half_bits(acc[a][b][r]);
        }
      }
}

// Y = fp16(sum over z of part[z]), summed in z order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            uint16_t* __restrict__ Y, int64_t MN, int splits) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < MN; i += (int64_t)gridDim.x * 256) {
    float v = part[i];
    for (int z = 1; z < splits; ++z) v += part[(size_t)z * MN + i];
    Y[i] = half_bits(v);
  }
}

// Y of the tail tiles = fp16(sum over the tsplit partials), in piece order.
// Grid: (XCD, tail tile of that XCD, 16 element chunks).
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
  for (int e = blockIdx.z * 256 + threadIdx.x; e < BM * BN; e += 256 * gridDim.z) {
    const int r = e / BN, c = e - r * BN;
    if (m0 + r < M && n0 + c < N) {
      const size_t o = (size_t)(m0 + r) * N + n0 + c;
      float v = part[o];
      for (int z = 1; z < tsplit; ++z) v += part[(size_t)z * MN + o];
      Y[o] = half_bits(v);
    }
  }
}

struct Config {
  int bm, bn, splits;
  int tsplit, full_x;  // tail split (1: none); tiles per XCD in its full rounds
};

// Pick the tile shape that keeps the most of the GPU's workgroup slots busy
// over whole rounds, weighted by how efficiently the shape uses LDS bandwidth
// per MFMA.  K is split (needs the workspace) only when the tiles cannot
// fill every slot once: then the smallest split reaching ~80 % of the slots.
#ifndef TKQ_PREFILL_SPLIT_SCORE
#define TKQ_PREFILL_SPLIT_SCORE 1
#endif
Config choose(int64_t M, int64_t N, int64_t K, int cus, int64_t ws_floats) {
  struct Cand {
    int bm, bn, per_cu;
    double eff;
  };
#ifndef TKQ_PREFILL_BIG
#define TKQ_PREFILL_BIG 0.5  // weight of the 128x256 / 256x128 tiles (measured slower: one wave per SIMD)
#endif
  const Cand cands[] = {{128, 256, 1, TKQ_PREFILL_BIG}, {256, 128, 1, TKQ_PREFILL_BIG}, {128, 128, 2, 1.0},
                        {128, 64, 2, 0.8},           {64, 128, 2, 0.8},           {64, 64, 4, 0.55}};
  const int64_t ksteps = (K + BK - 1) / BK;
  Config best = {128, 128, 1, 1, 0};
  double best_score = -1.0;
  for (const Cand& c : cands) {
    const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const int64_t slots = (int64_t)cus * c.per_cu;
#if TKQ_PREFILL_SPLIT_SCORE
    // with a workspace, a shape that leaves slots idle may split K: score the
    // pieces (s the smallest split that fills 80 % of the slots, as below)
    int s = 1;
    if (tiles < slots) {
      for (int t = 2; t <= 8; ++t) {
        if ((int64_t)t * M * N > ws_floats || t > ksteps / 4) break;
        s = t;
        if (tiles * t * 5 >= slots * 4) break;
      }
    }
    const int64_t items = tiles * s;
#else
    const int64_t items = tiles;
#endif
    const int64_t rounds = (items + slots - 1) / slots;
    const double score = double(items) / double(rounds * slots) * c.eff;
    if (score > best_score + 1e-9) {
      best_score = score;
      best = {c.bm, c.bn, 1, 1, 0};
    }
  }
  const int64_t tiles = ((M + best.bm - 1) / best.bm) * ((N + best.bn - 1) / best.bn);
  const int64_t slots = (int64_t)cus * (best.bm * best.bn > 128 * 128 ? 1 : best.bm * best.bn >= 128 * 64 ? 2 : 4);
  if (tiles < slots) {
    for (int s = 2; s <= 8; ++s) {
      if ((int64_t)s * M * N > ws_floats || s > ksteps / 4) break;
      best.splits = s;
      if (tiles * s * 5 >= slots * 4) break;
    }
  } else if (cus % kXcds == 0) {
    // Tail split: the rounds are those of the largest XCD range; every XCD
    // cuts the tiles after its full rounds (at most `last`) into s pieces,
    // the largest s with s * last within one round of slots.
    const int64_t sx = slots / kXcds, tiles_x = tiles / kXcds + (tiles % kXcds ? 1 : 0);
    const int64_t rounds = (tiles_x + sx - 1) / sx;
    const int64_t last = tiles_x - (rounds - 1) * sx;
#ifndef TKQ_PREFILL_TAIL
#define TKQ_PREFILL_TAIL 1
#endif
    for (int s = 4; s >= 2 && TKQ_PREFILL_TAIL; --s) {
      if (last * s <= sx && (int64_t)s * M * N <= ws_floats && s <= ksteps / 4) {
        best.tsplit = s;
        best.full_x = (int)((rounds - 1) * sx);
        break;
      }
    }
  }
  return best;
}

template <int BM, int BN>
void launch_tile(int64_t M, int64_t N, int64_t K, const Config& c, const uint32_t* codes, const uint32_t* meta,
                 const uint16_t* X, uint16_t* Y, float* part, hipStream_t stream) {
  const int64_t ksteps = (K + BK - 1) / BK;
  const int64_t T = ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
  if (c.tsplit > 1) {
    // per XCD: the full-round tiles, then tsplit pieces of each remaining
    // tile; grid = 8 x the largest XCD's item count
    const int64_t tiles_x = T / kXcds + (T % kXcds ? 1 : 0);
    const int64_t items = c.full_x + (tiles_x - c.full_x) * c.tsplit;
    const int per_piece = (int)((ksteps + c.tsplit - 1) / c.tsplit);
    hipLaunchKernelGGL((prefill_kernel<BM, BN>), dim3((uint32_t)(items * kXcds)), dim3(256), 0, stream, X, codes,
                       meta, Y, part, (int)M, (int)N, (int)K, per_piece, c.tsplit, c.full_x);
    return;
  }
  const int per_split = (int)((ksteps + c.splits - 1) / c.splits);
  const dim3 grid((uint32_t)(T * c.splits));
  hipLaunchKernelGGL((prefill_kernel<BM, BN>), grid, dim3(256), 0, stream, X, codes, meta, Y, part, (int)M,
                     (int)N, (int)K, per_split, 1, 0);
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
  if (c.bm == 128 && c.bn == 256) launch_tile<128, 256>(M, N, K, c, codes, meta, X, Y, part, stream);
  else if (c.bm == 256) launch_tile<256, 128>(M, N, K, c, codes, meta, X, Y, part, stream);
  else if (c.bm == 128 && c.bn == 128) launch_tile<128, 128>(M, N, K, c, codes, meta, X, Y, part, stream);
  else if (c.bm == 128) launch_tile<128, 64>(M, N, K, c, codes, meta, X, Y, part, stream);
  else if (c.bn == 128) launch_tile<64, 128>(M, N, K, c, codes, meta, X, Y, part, stream);
  else launch_tile<64, 64>(M, N, K, c, codes, meta, X, Y, part, stream);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (c.tsplit > 1) {
    const int64_t T = ((N + c.bn - 1) / c.bn) * ((M + c.bm - 1) / c.bm);
    const int64_t last = T / kXcds + (T % kXcds ? 1 : 0) - c.full_x;
    hipLaunchKernelGGL(tail_reduce_kernel, dim3(kXcds, (uint32_t)last, 16), dim3(256), 0, stream, workspace, Y,
                       (int)M, (int)N, c.bm, c.bn, c.tsplit, c.full_x);
    return hipGetLastError();
  }
  if (c.splits == 1) return e;
  const int64_t MN = M * N;
  int64_t blocks = (MN + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, workspace, Y, MN,
                     c.splits);
  return hipGetLastError();
}

}  // namespace tkq

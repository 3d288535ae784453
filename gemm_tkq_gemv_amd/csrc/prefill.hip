// Prefill GEMM over int4 g128 weights for gfx950: Y = X . dequant(W)^T.
//
// With M >= 64 tokens per weight the product is a dense contraction (the
// Whetstone README, "Prior art": the binary/bit paths only pay off in prefill
// or speculative verification, where the regime is compute-bound), so this is
// the one place the library uses the matrix cores.  As in TKintegers K5
// ("What is K5?"), tiles of low-bit codes are expanded to fp16 operands and
// multiplied with fp32 accumulation:
//
//  * A workgroup (4 wave64s, 2 x 2) owns a 128 x 128 tile of Y and walks K in
//    steps of 128 = one quantization group, so each weight row of the step
//    has exactly one (scale, zero) pair.
//  * Per step: X (fp16) is copied to LDS as is; the int4 codes are unpacked
//    with the fp16 magic-number trick, shifted by the zero point (exact small
//    integers) and multiplied by the fp16 scale (one fp16 rounding), then
//    written to LDS.  Rows are padded by 16 bytes against bank conflicts.
//  * Each wave computes a 64 x 64 sub-tile as 2 x 2 v_mfma_f32_32x32x16_f16.
//  * fp32 accumulators are rounded to fp16 (nearest even) on store.
#include "device_common.h"
#include "kernels.h"

namespace tkq {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDSW = BK + 8;  // halfs per LDS row (16 bytes of padding)
constexpr uint32_t kMagic = 0x64006400u;

__device__ __forceinline__ uint32_t dq(uint32_t field, h2 zoff, h2 s) {
  // field = two nibbles at bits [0,4) and [16,20): (q_a, q_b) -> s * (q - z)
  const h2 h = as_h2(field | kMagic) - zoff;
  return __builtin_bit_cast(uint32_t, h * s);
}

__global__ __launch_bounds__(256) void prefill_kernel(const uint16_t* __restrict__ X,
                                                      const uint32_t* __restrict__ codes,
                                                      const uint32_t* __restrict__ meta,
                                                      uint16_t* __restrict__ Y, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) _Float16 xs[BM * LDSW];
  __shared__ __attribute__((aligned(16))) _Float16 ws[BN * LDSW];

  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int mrows = min(BM, M - m0), nrows = min(BN, N - n0);
  const uint32_t xrow = (uint32_t)K * 2u, crow = (uint32_t)K / 2u, mrow = (uint32_t)(K / 128) * 4u;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X + (size_t)m0 * K, (uint32_t)mrows * xrow);
  const __amdgpu_buffer_rsrc_t cr = make_rsrc((const char*)codes + (size_t)n0 * crow, (uint32_t)nrows * crow);
  const __amdgpu_buffer_rsrc_t mr = make_rsrc((const char*)meta + (size_t)n0 * mrow, (uint32_t)nrows * mrow);

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += BK) {
    u32x4 xv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = i * 256 + tid, r = idx >> 4, c = idx & 15;
      xv[i] = load16(xr, (uint32_t)r * xrow + (uint32_t)k0 * 2u + (uint32_t)c * 16u);
    }
    u32x4 wv[2];
    uint32_t mv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = i * 256 + tid, r = idx >> 2, c = idx & 3;
      wv[i] = load16_nt(cr, (uint32_t)r * crow + (uint32_t)k0 / 2u + (uint32_t)c * 16u);
      mv[i] = load4(mr, (uint32_t)r * mrow + (uint32_t)(k0 / 128) * 4u);
    }
    __syncthreads();  // the previous step's MFMA operands have been read
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = i * 256 + tid, r = idx >> 4, c = idx & 15;
      *reinterpret_cast<u32x4*>(&xs[r * LDSW + c * 8]) = xv[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = i * 256 + tid, r = idx >> 2, c = idx & 3;
      const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(mv[i] & 0xFFFFu));
      const _Float16 z = __builtin_bit_cast(_Float16, (uint16_t)(mv[i] >> 16));
      const h2 ss = {s, s};
      const _Float16 zo = (_Float16)1024.0f + z;  // exact: z is an integer 0..15
      const h2 zoff = {zo, zo};
      u32x4 out[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t v = wv[i][w];
        const uint32_t a = dq(v & 0x000F000Fu, zoff, ss);          // (w0, w4)
        const uint32_t b = dq((v >> 4) & 0x000F000Fu, zoff, ss);   // (w1, w5)
        const uint32_t cc = dq((v >> 8) & 0x000F000Fu, zoff, ss);  // (w2, w6)
        const uint32_t d = dq((v >> 12) & 0x000F000Fu, zoff, ss);  // (w3, w7)
        out[w][0] = __builtin_amdgcn_perm(b, a, 0x05040100u);   // (w0, w1)
        out[w][1] = __builtin_amdgcn_perm(d, cc, 0x05040100u);  // (w2, w3)
        out[w][2] = __builtin_amdgcn_perm(b, a, 0x07060302u);   // (w4, w5)
        out[w][3] = __builtin_amdgcn_perm(d, cc, 0x07060302u);  // (w6, w7)
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) *reinterpret_cast<u32x4*>(&ws[r * LDSW + c * 32 + w * 8]) = out[w];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      half8 a[2], b[2];
      const int kk = ks + (lane >> 5) * 8;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *reinterpret_cast<const half8*>(&xs[(wm + t * 32 + (lane & 31)) * LDSW + kk]);
        b[t] = *reinterpret_cast<const half8*>(&ws[(wn + t * 32 + (lane & 31)) * LDSW + kk]);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[p][q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[p], b[q], acc[p][q], 0, 0, 0);
    }
  }

  // D layout of a 32x32 fp32 accumulator: register r of lane l holds row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = wm + p * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int j = wn + q * 32 + (lane & 31);
        if (i < mrows && j < nrows) Y[(size_t)(m0 + i) * N + n0 + j] = half_bits(acc[p][q][r]);
      }
}

}  // namespace

hipError_t launch_prefill(int64_t M, int64_t N, int64_t K, const uint32_t* codes,
                          const uint32_t* meta, const uint16_t* X, uint16_t* Y, hipStream_t stream) {
  const dim3 grid((uint32_t)((N + BN - 1) / BN), (uint32_t)((M + BM - 1) / BM));
  hipLaunchKernelGGL(prefill_kernel, grid, dim3(256), 0, stream, X, codes, meta, Y, (int)M, (int)N,
                     (int)K);
  return hipGetLastError();
}

}  // namespace tkq

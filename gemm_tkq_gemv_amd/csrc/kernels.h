// Internal launch interface between the C-ABI layer (tkq_api.hip) and the
// kernel translation units.  Every launcher assumes arguments that the C-ABI
// layer has already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tkq.h"

namespace tkq {

constexpr int kFmtInt4 = TKQ_FMT_INT4_G128;
constexpr int kFmtK5 = TKQ_FMT_K5_G128;
constexpr int kFmtTern = TKQ_FMT_TERN_G128;
constexpr int kFmtBin = TKQ_FMT_BIN;
constexpr int kFmtHier = TKQ_FMT_INT4_HIER_G32;
constexpr int kFmtInt2 = TKQ_FMT_INT2_G128;
constexpr int kFmtInt3 = TKQ_FMT_INT3_G128;

// Work decomposition of one GEMV, packed into tkq_gemv_desc::shape.
struct GemvShape {
  int lanes_log2;  // lanes cooperating on one row (1..64)
  int passes;      // 16-byte chunks each lane reads per row
  int kslices;     // waves that split one row's K range (1, 2 or 4)
};
__host__ __device__ inline int pack_shape(GemvShape s) { return s.lanes_log2 | (s.passes << 4) | (s.kslices << 16); }
__host__ __device__ inline GemvShape unpack_shape(int v) { return {v & 15, (v >> 4) & 4095, (v >> 16) & 15}; }

// Weights carried by one 16-byte chunk of codes, per coding.
inline int weights_per_chunk(int fmt) {
  switch (fmt) {
    case kFmtInt4: return 32;
    case kFmtHier: return 32;
    case kFmtK5: return 16;
    case kFmtTern: return 64;
    case kFmtInt2: return 64;
    case kFmtInt3: return 128;
    case kFmtBin: return 128;
  }
  return 0;
}

// Bytes of codes per chunk (one lane's unit of a row): 16, or 48 for int3
// (three 16-byte planes).
inline int chunk_bytes(int fmt) { return fmt == kFmtInt3 ? 48 : 16; }

// Largest row tile of one GEMV workgroup (bounds the k-slice LDS buffer).
constexpr int kGemvMaxTileRows = 1024;

// Row steps a wave keeps in flight per loop iteration for J passes: deep
// enough that every CU has ~100 KB of loads outstanding.  Used by the kernel
// and by the planner (tile heights are multiples of it).
__host__ __device__ constexpr int gemv_unroll(int passes) { return passes == 1 ? 4 : (passes == 2 ? 2 : 1); }

// int4 g128 GEMV: dynamic LDS of a tile of `rows` rows of K columns -- x
// (two copies when K / 128 is odd) and eight fp32 slots per row -- and the
// limit it is held to (160 KB per workgroup less the static part).
constexpr int kInt4MaxLds = 160 * 1024 - 64;
__host__ __device__ constexpr int64_t int4_lds_bytes(int K, int rows) {
  return int64_t((K / 128) % 2 ? 2 * (K / 128) : K / 128) * 256 + int64_t(rows) * 32;
}

// Largest `passes` value each kernel variant supports (x stays in registers).
int gemv_max_passes(int fmt);
// jmax: largest `passes` among the descriptors (selects the kernel variant).
// target >= 0: also store the largest output key of each of descriptor
// `target`'s row tiles into slots (scratch of one uint64 per tile of the
// launch) and, when token is not null, select the largest into *token.
hipError_t launch_gemv(int fmt, int jmax, const tkq_gemv_desc* dev_descs, int count, int64_t tiles,
                       int target, int32_t* token, uint64_t* slots, hipStream_t stream);

// Multi-token GEMV (int4 g128, or int4-hier-g32 when hier, M = 1..16): one
// workgroup (4 waves of 16 rows) per 64-row tile; descriptors prepared by
// tkq_gemm_small_prepare.
constexpr int kSmallTileRows = 64;
constexpr int kSmallMaxM = 16;
hipError_t launch_small_m(const tkq_gemv_desc* dev_descs, int count, int64_t tiles, int M, bool hier,
                          hipStream_t stream);

// Low-bit KV cache (pages of 128 tokens, head dimension 128) and decode.
constexpr int kKvPage = 128, kKvDim = 128, kKvPageBytes = 17408, kKvWaves = 4, kKvMaxGroup = 8;
// lens: device int32 [B] of valid tokens per sequence (clamped to [0, T]), or
// nullptr for all T.
hipError_t launch_kv_pack(const uint16_t* K, const uint16_t* V, const int32_t* lens, int B, int T, int Hk,
                          uint32_t* cache, hipStream_t stream);
int kv_splits(int B, int H, int Hk, int T, int cus, int* pages_per_split);
// ws: the splits' partials; counters: one zero-initialised uint32 per
// (sequence, head group), left at zero by every completed call.
hipError_t launch_kv_decode(const uint16_t* q, const uint32_t* cache, const int32_t* lens, int B, int H, int Hk,
                            int T, float sm_scale, uint16_t* out, float* ws, uint32_t* counters, int splits,
                            int pages_per_split, hipStream_t stream);

hipError_t launch_pack(int fmt, const float* W, int64_t N, int64_t K, void* codes, void* meta,
                       hipStream_t stream);

// Byte offset of the per-row fp16 pairs in an int4-hier-g32 metadata block.
__host__ __device__ inline int64_t hier_row_offset(int64_t N, int64_t K) { return (N * (K / 32) + 15) / 16 * 16; }

hipError_t launch_prefill(int64_t M, int64_t N, int64_t K, const uint32_t* codes, const uint32_t* meta,
                          const uint16_t* X, uint16_t* Y, float* workspace, int64_t workspace_bytes,
                          hipStream_t stream);

// Greedy selection with head rescore: one workgroup of 1024 threads.
// rescore_capacity: keys the candidate collection may hold (k shares).
int64_t rescore_capacity(int64_t n, int k);
hipError_t launch_head_rescore(const uint16_t* logits, int64_t n, const uint16_t* head, const uint16_t* x,
                               int64_t K, int k, int32_t* token, int32_t* cand, float* cand_logits,
                               hipStream_t stream);

// The same selection over a grouped GEMV's target, from the per-tile keys the
// greedy variant stored in slots (launch_gemv with token = nullptr first).
hipError_t launch_gemv_rescore(const tkq_gemv_desc* dev_descs, int count, int target, int64_t tiles,
                               const uint64_t* slots, const uint16_t* head, int k, int32_t* token, int32_t* cand,
                               float* cand_logits, hipStream_t stream);

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* out, hipStream_t stream);

}  // namespace tkq

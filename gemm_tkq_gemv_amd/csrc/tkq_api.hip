// C-ABI entry points of libtkq: host-side validation, the GEMV work planner,
// and the kernel launches.  Every check runs on the host before any HIP call;
// on failure nothing is enqueued.
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "kernels.h"

namespace {

thread_local int g_last_hip_error = 0;
constexpr int32_t kPlanMagic = 0x746b7131;   // "tkq1": tkq_gemv_prepare
constexpr int32_t kSmallMagic = 0x746b7132;  // "tkq2": tkq_gemm_small_prepare
constexpr int64_t kMaxWeights = int64_t(1) << 39;
// Planner parameters per coding (measured on MI355X, interleaved runs):
//  tile   bytes of codes one wave streams per large tile: large enough to
//         amortise the per-tile setup (descriptor search, x slice,
//         constants);
//  small  bytes per wave of the small tiles used over the last `tail` bytes
//         of a sweep, so the final workgroups finish close together (about
//         two rounds of small tiles for every workgroup slot of a 256-CU
//         part);
//  prefer_passes  on equal lane utilisation, the pass count to prefer: more
//         passes = more rows per wave step = fewer cross-lane reductions per
//         row, at the cost of x registers.
//  max_passes  cap on passes: the launch's kernel variant is sized for the
//         largest pass count of its matrices, so one long-K matrix would set
//         the register budget (and occupancy) of the whole sweep.
struct PlanParams {
  int prefer_passes, max_passes;
  int64_t tile, small, tail;
};
PlanParams plan_params(int fmt) {
  if (fmt == TKQ_FMT_INT4_G128 || fmt == TKQ_FMT_INT4_HIER_G32) return {2, 4, 48 << 10, 4 << 10, 60 << 20};
  if (fmt == TKQ_FMT_TERN_G128 || fmt == TKQ_FMT_INT2_G128) return {1, 2, 24 << 10, 4 << 10, 40 << 20};
  if (fmt == TKQ_FMT_INT3_G128) return {1, 1, 24 << 10, 4 << 10, 40 << 20};
  return {1, 8, 24 << 10, 4 << 10, 40 << 20};
}
constexpr int kMaxTileRows = tkq::kGemvMaxTileRows;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return TKQ_OK;
  g_last_hip_error = (int)e;
  return TKQ_EHIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool known_fmt(int fmt) {
  return fmt == TKQ_FMT_INT4_G128 || fmt == TKQ_FMT_K5_G128 || fmt == TKQ_FMT_TERN_G128 ||
         fmt == TKQ_FMT_BIN || fmt == TKQ_FMT_INT4_HIER_G32 || fmt == TKQ_FMT_INT2_G128 ||
         fmt == TKQ_FMT_INT3_G128;
}

// Column unit of a coding's GEMV (its group size, or one code word).
int k_unit(int fmt) { return fmt == TKQ_FMT_INT4_HIER_G32 ? 32 : 128; }

// Largest K each GEMV handles: int4 keeps x in LDS (64 KB at K = 32768); the
// other codings keep x in registers, chunks per row <= 4 k-slices x 64 lanes
// x the planner's pass cap.
int64_t gemv_max_k(int fmt) {
  if (fmt == TKQ_FMT_INT4_G128) return 32768;  // x in LDS: two copies of K = 32640 still fit
  return int64_t(4) * 64 * std::min(tkq::gemv_max_passes(fmt), plan_params(fmt).max_passes) *
         tkq::weights_per_chunk(fmt);
}

int check_matrix(const float* W, int64_t N, int64_t K, int64_t kunit) {
  if (!W || N < 1 || K < 1) return TKQ_EINVAL;
  if (K % kunit || K > TKQ_MAX_K || N > INT32_MAX || N * K > kMaxWeights) return TKQ_ESHAPE;
  if (!aligned16(W)) return TKQ_EALIGN;
  return TKQ_OK;
}

int pack_common(int fmt, const float* W, int64_t N, int64_t K, void* codes, void* meta,
                bool need_meta, int64_t kunit, void* stream) {
  int st = check_matrix(W, N, K, kunit);
  if (st) return st;
  if (!codes || (need_meta && !meta)) return TKQ_EINVAL;
  if (!aligned16(codes) || (need_meta && !aligned16(meta))) return TKQ_EALIGN;
  return hip_status(tkq::launch_pack(fmt, W, N, K, codes, meta, (hipStream_t)stream));
}

// Choose lanes-per-row, passes and k-slices for one GEMV: the decomposition
// with the fewest idle lane-chunk slots (16-byte chunks per row over
// k-slices x lanes x passes).
tkq::GemvShape choose_shape(int fmt, int K) {
  // int4: units of eight lanes walk whole rows group by group (the kernel
  // has no passes or k-slices to choose).
  if (fmt == TKQ_FMT_INT4_G128) return {3, K / 128, 1};
  const int prefer = plan_params(fmt).prefer_passes;
  const int C = K / tkq::weights_per_chunk(fmt);
  const int jmax = std::min(tkq::gemv_max_passes(fmt), plan_params(fmt).max_passes);
  tkq::GemvShape best = {6, 0, 0};
  double best_util = -1.0;
  for (int S : {1, 2, 4}) {
    const int Cs = (C + S - 1) / S;
    for (int lg = 6; lg >= 0; --lg) {
      const int L = 1 << lg;
      const int J = (Cs + L - 1) / L;
      if (J > jmax) continue;
      const double util = double(C) / double(S * L * J);
      // Ties: fewer k-slices, then the pass count closest to the preferred one.
      const int dj = J > prefer ? J - prefer : prefer - J;
      const int db = best.passes > prefer ? best.passes - prefer : prefer - best.passes;
      const bool better = util > best_util + 1e-12 ||
                          (util > best_util - 1e-12 &&
                           (S < best.kslices || (S == best.kslices && dj < db)));
      if (better) {
        best = {lg, J, S};
        best_util = util;
      }
    }
  }
  return best;
}

// int4 g128: a tile is 32 units of R rows, R ~ the target bytes per wave over
// eight units; R even when a row has an odd number of groups (units then
// start on 128-byte boundaries), and the tile's LDS (x, metadata, row slots)
// within the per-workgroup limit.
int int4_rows_per_tile(int K, int64_t target) {
  const int G = K / 128;
  const int64_t row_bytes = int64_t(K) / 2;
  int R = (int)std::max<int64_t>(1, (target + 8 * row_bytes - 1) / (8 * row_bytes));
  R = std::min(R, tkq::kGemvMaxTileRows / 32);
  if ((G & 1) && R > 1) R &= ~1;
  while (R > 1 && tkq::int4_lds_bytes(K, 32 * R) > tkq::kInt4MaxLds) R -= (G & 1) && R > 2 ? 2 : 1;
  return 32 * R;
}

int rows_per_tile(int fmt, int N, int K, tkq::GemvShape sh, int64_t kTileTargetBytes) {
  if (fmt == TKQ_FMT_INT4_G128) return int4_rows_per_tile(K, kTileTargetBytes);
  const int C = K / tkq::weights_per_chunk(fmt);
  const int Cs = (C + sh.kslices - 1) / sh.kslices;
  const int P = 64 >> sh.lanes_log2;       // rows per wave step
  const int RG = 4 / sh.kslices;           // row groups per workgroup
  const int U = fmt == TKQ_FMT_INT4_G128 ? 1 : tkq::gemv_unroll(sh.passes);  // steps per loop iteration
  const int64_t step_bytes = int64_t(P) * Cs * tkq::chunk_bytes(fmt);
  int64_t steps = (kTileTargetBytes + step_bytes - 1) / step_bytes;
  const int64_t need = ((int64_t(N) + RG - 1) / RG + P - 1) / P;  // steps to cover N
  if (steps > need) steps = need;
  steps = ((steps + U - 1) / U) * U;
  while (steps > U && int64_t(RG) * P * steps > kMaxTileRows) steps -= U;
  return (int)(int64_t(RG) * P * steps);
}

// Scratch of tkq_gemv_argmax_static: one 64-bit key per row tile of a
// launch, in device memory that each GPU the library runs on holds until the
// process ends (TKQ_STATIC_SLOTS * 8 bytes = 512 KB).  Host code never uses
// the array's name as an address: the address on each device comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) uint64_t scratch[TKQ_STATIC_SLOTS];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
uint64_t* g_scratch_ptr[kMaxDevices] = {};

// This thread's current device's copy of `scratch`.
int static_scratch(uint64_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return TKQ_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    g_scratch_ptr[dev] = static_cast<uint64_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return TKQ_OK;
}

}  // namespace

extern "C" {

int tkq_version(void) { return TKQ_VERSION; }

const char* tkq_strerror(int status) {
  switch (status) {
    case TKQ_OK: return "success";
    case TKQ_EINVAL: return "invalid argument (null pointer, non-positive size or count)";
    case TKQ_ESHAPE: return "unsupported shape (K not a multiple of the format's unit, or too large)";
    case TKQ_EALIGN: return "device pointer not 16-byte aligned";
    case TKQ_EFORMAT: return "unknown or mixed weight format";
    case TKQ_EHIP: return "HIP call failed (see tkq_last_hip_error)";
    case TKQ_EPLAN: return "plan was not produced by tkq_gemv_prepare";
  }
  return "unknown status";
}

int tkq_last_hip_error(void) { return g_last_hip_error; }

int tkq_pack_int4_g128(const float* W, int64_t N, int64_t K, uint32_t* codes, uint32_t* meta,
                       void* stream) {
  return pack_common(TKQ_FMT_INT4_G128, W, N, K, codes, meta, true, 128, stream);
}

int tkq_pack_k5(const float* W, int64_t N, int64_t K, uint8_t* codes, uint16_t* scale,
                void* stream) {
  return pack_common(TKQ_FMT_K5_G128, W, N, K, codes, scale, true, 128, stream);
}

int tkq_pack_tern_g128(const float* W, int64_t N, int64_t K, uint32_t* codes, uint16_t* scale,
                       void* stream) {
  return pack_common(TKQ_FMT_TERN_G128, W, N, K, codes, scale, true, 128, stream);
}

int tkq_pack_bin(const float* W, int64_t N, int64_t K, uint32_t* bits, void* stream) {
  return pack_common(TKQ_FMT_BIN, W, N, K, bits, nullptr, false, 32, stream);
}

int tkq_pack_int2_g128(const float* W, int64_t N, int64_t K, uint32_t* codes, uint32_t* meta,
                       void* stream) {
  return pack_common(TKQ_FMT_INT2_G128, W, N, K, codes, meta, true, 128, stream);
}

int tkq_pack_int3_g128(const float* W, int64_t N, int64_t K, uint32_t* codes, uint32_t* meta,
                       void* stream) {
  return pack_common(TKQ_FMT_INT3_G128, W, N, K, codes, meta, true, 128, stream);
}

int tkq_pack_int4_hier_g32(const float* W, int64_t N, int64_t K, uint32_t* codes, uint8_t* meta,
                           void* stream) {
  return pack_common(TKQ_FMT_INT4_HIER_G32, W, N, K, codes, meta, true, 32, stream);
}

int64_t tkq_hier_meta_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 32 || K % 32 || K > TKQ_MAX_K || N > INT32_MAX) return -1;
  return tkq::hier_row_offset(N, K) + 4 * N;
}

int tkq_gemv_prepare(tkq_gemv_desc* descs, int32_t count, tkq_gemv_plan* plan) {
  if (!descs || !plan || count < 1) return TKQ_EINVAL;
  const int fmt = descs[0].fmt;
  if (!known_fmt(fmt)) return TKQ_EFORMAT;
  for (int32_t i = 0; i < count; ++i) {
    const tkq_gemv_desc& d = descs[i];
    if (d.fmt != fmt) return TKQ_EFORMAT;
    if (d.N < 1 || d.K < 1 || !d.codes || !d.x || !d.y) return TKQ_EINVAL;
    if (fmt != TKQ_FMT_BIN && !d.meta) return TKQ_EINVAL;
    if (d.K % k_unit(fmt) || d.K > gemv_max_k(fmt) || int64_t(d.N) * d.K > kMaxWeights) return TKQ_ESHAPE;
    if (!aligned16(d.codes) || !aligned16(d.x) || !aligned16(d.y) ||
        (fmt != TKQ_FMT_BIN && !aligned16(d.meta)))
      return TKQ_EALIGN;
  }
  // Sweep position where the small-tile tail begins.
  int64_t total = 0;
  for (int32_t i = 0; i < count; ++i)
    total += int64_t(descs[i].N) * (descs[i].K / tkq::weights_per_chunk(fmt)) * tkq::chunk_bytes(fmt);
  const PlanParams pp = plan_params(fmt);
  const int64_t tail_start = total > pp.tail ? total - pp.tail : 0;

  int64_t work = 0, pos = 0;
  int jmax = 1;
  for (int32_t i = 0; i < count; ++i) {
    tkq_gemv_desc& d = descs[i];
    const tkq::GemvShape sh = choose_shape(fmt, d.K);
    if (sh.passes < 1) return TKQ_ESHAPE;
    const int big = rows_per_tile(fmt, d.N, d.K, sh, pp.tile);
    const int small = rows_per_tile(fmt, d.N, d.K, sh, pp.small);
    const int64_t row_bytes = int64_t(d.K / tkq::weights_per_chunk(fmt)) * tkq::chunk_bytes(fmt);
    // rows above the tail start get large tiles
    int64_t big_rows = 0;
    if (pos + d.N * row_bytes <= tail_start) big_rows = d.N;
    else if (pos < tail_start) big_rows = (tail_start - pos + row_bytes - 1) / row_bytes;
    const int64_t nbig = (big_rows + big - 1) / big;
    const int64_t rest = int64_t(d.N) - nbig * big;
    const int64_t tiles = nbig + (rest > 0 ? (rest + small - 1) / small : 0);
    if (work + tiles > INT32_MAX) return TKQ_ESHAPE;
    d.work0 = (int32_t)work;
    d.big_tiles = (int32_t)nbig;
    d.rows_per_tile = big;
    d.shape = tkq::pack_shape(sh);
    d.small_rows = small;
    work += tiles;
    pos += d.N * row_bytes;
    if (fmt == TKQ_FMT_INT4_G128) {  // the variant is the launch's LDS bytes
      const int64_t lds = tkq::int4_lds_bytes(d.K, big);
      if (lds > jmax) jmax = (int)lds;
    } else if (sh.passes > jmax) {
      jmax = sh.passes;
    }
  }
  plan->fmt = fmt;
  plan->count = count;
  plan->tiles = work;
  plan->variant = jmax;
  plan->magic = kPlanMagic;
  plan->reserved = 0;
  return TKQ_OK;
}

static int check_plan(const tkq_gemv_plan* plan, const tkq_gemv_desc* dev_descs) {
  if (!plan || !dev_descs) return TKQ_EINVAL;
  if (plan->magic != kPlanMagic || !known_fmt(plan->fmt) || plan->count < 1 || plan->tiles < 1 ||
      plan->tiles > INT32_MAX || plan->variant < 1 ||
      plan->variant > (plan->fmt == TKQ_FMT_INT4_G128 ? tkq::kInt4MaxLds : tkq::gemv_max_passes(plan->fmt)))
    return TKQ_EPLAN;
  if (!aligned16(dev_descs)) return TKQ_EALIGN;
  return TKQ_OK;
}

int tkq_gemv(const tkq_gemv_plan* plan, const tkq_gemv_desc* dev_descs, void* stream) {
  const int st = check_plan(plan, dev_descs);
  if (st) return st;
  return hip_status(tkq::launch_gemv(plan->fmt, plan->variant, dev_descs, plan->count, plan->tiles, -1,
                                     nullptr, nullptr, (hipStream_t)stream));
}

int tkq_gemv_argmax(const tkq_gemv_plan* plan, const tkq_gemv_desc* dev_descs, int32_t target,
                    int32_t* token, uint64_t* slots, int64_t scratch_bytes, void* stream) {
  const int st = check_plan(plan, dev_descs);
  if (st) return st;
  if (!token || !slots || target < 0 || target >= plan->count) return TKQ_EINVAL;
  if (scratch_bytes < 8 * plan->tiles) return TKQ_EINVAL;
  if ((reinterpret_cast<uintptr_t>(token) & 3u) || !aligned16(slots)) return TKQ_EALIGN;
  return hip_status(tkq::launch_gemv(plan->fmt, plan->variant, dev_descs, plan->count, plan->tiles,
                                     target, token, slots, (hipStream_t)stream));
}

int tkq_gemv_argmax_static(const tkq_gemv_plan* plan, const tkq_gemv_desc* dev_descs, int32_t target,
                           int32_t* token, void* stream) {
  const int st = check_plan(plan, dev_descs);
  if (st) return st;
  if (!token || target < 0 || target >= plan->count) return TKQ_EINVAL;
  if (plan->tiles > TKQ_STATIC_SLOTS) return TKQ_ESHAPE;
  if (reinterpret_cast<uintptr_t>(token) & 3u) return TKQ_EALIGN;
  uint64_t* slots = nullptr;
  const int ss = static_scratch(&slots);
  if (ss) return ss;
  // Every slot the selection reads is written by the same launch (one per
  // tile of the target), so nothing needs clearing between calls.
  return hip_status(tkq::launch_gemv(plan->fmt, plan->variant, dev_descs, plan->count, plan->tiles,
                                     target, token, slots, (hipStream_t)stream));
}

int tkq_gemm_small_prepare(tkq_gemv_desc* descs, int32_t count, int32_t M, tkq_gemv_plan* plan) {
  if (!descs || !plan || count < 1 || M < 1) return TKQ_EINVAL;
  if (M > tkq::kSmallMaxM) return TKQ_ESHAPE;
  const int32_t fmt = descs[0].fmt;
  if (fmt != TKQ_FMT_INT4_G128 && fmt != TKQ_FMT_INT4_HIER_G32) return TKQ_EFORMAT;
  int64_t work = 0;
  for (int32_t i = 0; i < count; ++i) {
    tkq_gemv_desc& d = descs[i];
    if (d.fmt != fmt) return TKQ_EFORMAT;
    if (d.N < 1 || d.K < 1 || !d.codes || !d.meta || !d.x || !d.y) return TKQ_EINVAL;
    if (d.K % 128 || d.K > TKQ_MAX_K || int64_t(d.N) * d.K > kMaxWeights ||
        int64_t(M) * d.K * 2 > INT32_MAX || int64_t(M) * d.N * 2 > INT32_MAX)
      return TKQ_ESHAPE;
    if (!aligned16(d.codes) || !aligned16(d.meta) || !aligned16(d.x) || !aligned16(d.y)) return TKQ_EALIGN;
    const int64_t tiles = (int64_t(d.N) + tkq::kSmallTileRows - 1) / tkq::kSmallTileRows;
    if (work + tiles > INT32_MAX) return TKQ_ESHAPE;
    d.work0 = (int32_t)work;
    d.big_tiles = (int32_t)tiles;
    d.rows_per_tile = tkq::kSmallTileRows;
    d.shape = 0;
    d.small_rows = tkq::kSmallTileRows;
    work += tiles;
  }
  plan->fmt = fmt;
  plan->count = count;
  plan->tiles = work;
  plan->variant = M;
  plan->magic = kSmallMagic;
  plan->reserved = 0;
  return TKQ_OK;
}

int tkq_gemm_small(const tkq_gemv_plan* plan, const tkq_gemv_desc* dev_descs, void* stream) {
  if (!plan || !dev_descs) return TKQ_EINVAL;
  if (plan->magic != kSmallMagic || (plan->fmt != TKQ_FMT_INT4_G128 && plan->fmt != TKQ_FMT_INT4_HIER_G32) ||
      plan->count < 1 || plan->tiles < 1 ||
      plan->tiles > INT32_MAX || plan->variant < 1 || plan->variant > tkq::kSmallMaxM)
    return TKQ_EPLAN;
  if (!aligned16(dev_descs)) return TKQ_EALIGN;
  return hip_status(tkq::launch_small_m(dev_descs, plan->count, plan->tiles, plan->variant,
                                        plan->fmt == TKQ_FMT_INT4_HIER_G32, (hipStream_t)stream));
}

static int check_kv(int64_t B, int64_t H, int64_t Hk, int64_t T, int64_t D) {
  if (B < 1 || H < 1 || Hk < 1 || T < 1) return TKQ_EINVAL;
  if (D != tkq::kKvDim || T % tkq::kKvPage || H % Hk || B > 65535 || T > (int64_t(1) << 24) ||
      B * Hk * (T / tkq::kKvPage) * tkq::kKvPageBytes > (int64_t(1) << 40))
    return TKQ_ESHAPE;
  return TKQ_OK;
}

int64_t tkq_kv_cache_bytes(int32_t B, int32_t Hk, int32_t T) {
  if (check_kv(B, Hk, Hk, T, tkq::kKvDim)) return -1;
  return int64_t(B) * Hk * (T / tkq::kKvPage) * tkq::kKvPageBytes;
}

}  // extern "C"

namespace {
// Workspace of a decode: one arrival counter per (sequence, query head)
// first (so that a workspace zeroed once serves every later call with no
// more sequences x heads), then the splits' partials at a 16-byte boundary
// (one (m, l, o[128]) per head and split, at most one split per kKvWaves
// pages).
int64_t kv_counter_bytes(int32_t B, int32_t H) { return (int64_t(B) * H * 4 + 15) / 16 * 16; }
int64_t kv_partial_bytes(int32_t B, int32_t H, int32_t T) {
  const int64_t max_parts = (T / tkq::kKvPage + tkq::kKvWaves - 1) / tkq::kKvWaves * tkq::kKvWaves;
  return int64_t(B) * H * max_parts * (tkq::kKvDim + 2) * 4;
}

int kv_decode_common(const uint16_t* q, const uint32_t* cache, const int32_t* lens, int32_t B, int32_t H,
                     int32_t Hk, int32_t T, int32_t D, float sm_scale, uint16_t* out, float* workspace,
                     int64_t workspace_bytes, void* stream) {
  if (!q || !cache || !out || !workspace) return TKQ_EINVAL;
  const int st = check_kv(B, H, Hk, T, D);
  if (st) return st;
  if (!(sm_scale > 0.0f) || !(sm_scale < 1e30f)) return TKQ_EINVAL;
  if (workspace_bytes < tkq_kv_decode_workspace_bytes(B, H, Hk, T)) return TKQ_EINVAL;
  if (!aligned16(q) || !aligned16(cache) || !aligned16(out) || !aligned16(workspace)) return TKQ_EALIGN;
  if (lens && (reinterpret_cast<uintptr_t>(lens) & 3u)) return TKQ_EALIGN;
  int device = 0;
  hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &device) : hipGetDevice(&device);
  if (e != hipSuccess) return hip_status(e);
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_status(e);
  int pps = 1;
  const int splits = tkq::kv_splits(B, H, Hk, T, cus, &pps);
  uint32_t* counters = reinterpret_cast<uint32_t*>(workspace);
  float* parts = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + kv_counter_bytes(B, H));
  return hip_status(tkq::launch_kv_decode(q, cache, lens, B, H, Hk, T, sm_scale, out, parts, counters, splits, pps,
                                          (hipStream_t)stream));
}

int kv_pack_common(const uint16_t* K, const uint16_t* V, const int32_t* lens, int32_t B, int32_t T, int32_t Hk,
                   int32_t D, uint32_t* cache, void* stream) {
  if (!K || !V || !cache) return TKQ_EINVAL;
  const int st = check_kv(B, Hk, Hk, T, D);
  if (st) return st;
  if (!aligned16(K) || !aligned16(V) || !aligned16(cache)) return TKQ_EALIGN;
  if (lens && (reinterpret_cast<uintptr_t>(lens) & 3u)) return TKQ_EALIGN;
  return hip_status(tkq::launch_kv_pack(K, V, lens, B, T, Hk, cache, (hipStream_t)stream));
}
}  // namespace

extern "C" {

int64_t tkq_kv_decode_workspace_bytes(int32_t B, int32_t H, int32_t Hk, int32_t T) {
  if (check_kv(B, H, Hk, T, tkq::kKvDim)) return -1;
  return kv_counter_bytes(B, H) + kv_partial_bytes(B, H, T);
}

int tkq_kv_pack(const uint16_t* K, const uint16_t* V, int32_t B, int32_t T, int32_t Hk, int32_t D, uint32_t* cache,
                void* stream) {
  return kv_pack_common(K, V, nullptr, B, T, Hk, D, cache, stream);
}

int tkq_kv_pack_varlen(const uint16_t* K, const uint16_t* V, const int32_t* seqlens, int32_t B, int32_t T,
                       int32_t Hk, int32_t D, uint32_t* cache, void* stream) {
  if (!seqlens) return TKQ_EINVAL;
  return kv_pack_common(K, V, seqlens, B, T, Hk, D, cache, stream);
}

int tkq_kv_decode(const uint16_t* q, const uint32_t* cache, int32_t B, int32_t H, int32_t Hk, int32_t T, int32_t D,
                  float sm_scale, uint16_t* out, float* workspace, int64_t workspace_bytes, void* stream) {
  return kv_decode_common(q, cache, nullptr, B, H, Hk, T, D, sm_scale, out, workspace, workspace_bytes, stream);
}

int tkq_kv_decode_varlen(const uint16_t* q, const uint32_t* cache, const int32_t* seqlens, int32_t B, int32_t H,
                         int32_t Hk, int32_t T, int32_t D, float sm_scale, uint16_t* out, float* workspace,
                         int64_t workspace_bytes, void* stream) {
  if (!seqlens) return TKQ_EINVAL;
  return kv_decode_common(q, cache, seqlens, B, H, Hk, T, D, sm_scale, out, workspace, workspace_bytes, stream);
}

int tkq_gemm_prefill(int32_t fmt, int64_t M, int64_t N, int64_t K, const uint32_t* codes,
                     const uint32_t* meta, const uint16_t* X, uint16_t* Y, float* workspace,
                     int64_t workspace_bytes, void* stream) {
  if (fmt != TKQ_FMT_INT4_G128) return TKQ_EFORMAT;
  if (!codes || !meta || !X || !Y || M < 1 || N < 1 || K < 1 || workspace_bytes < 0 ||
      (workspace && workspace_bytes == 0))
    return TKQ_EINVAL;
  if (K % 128 || K > TKQ_MAX_K || M > INT32_MAX || N > INT32_MAX || N * K > kMaxWeights ||
      M * K > kMaxWeights || M * N > kMaxWeights || (M + 63) / 64 * ((N + 63) / 64) * 8 > INT32_MAX ||
      128 * K * 2 > INT32_MAX)
    return TKQ_ESHAPE;
  if (!aligned16(codes) || !aligned16(meta) || !aligned16(X) || !aligned16(Y) ||
      (workspace && !aligned16(workspace)))
    return TKQ_EALIGN;
  return hip_status(tkq::launch_prefill(M, N, K, codes, meta, X, Y, workspace,
                                        workspace ? workspace_bytes : 0, (hipStream_t)stream));
}

int tkq_head_rescore(const uint16_t* logits, int64_t n, const uint16_t* head, const uint16_t* x, int64_t K,
                     int32_t k, int32_t* token, int32_t* cand, float* cand_logits, void* stream) {
  if (!logits || !head || !x || !token || n < 1 || K < 1 || k < 1 || k > n) return TKQ_EINVAL;
  if (k > TKQ_RESCORE_MAX_K || n > INT32_MAX || K % 8 || K > TKQ_MAX_K ||
      tkq::rescore_capacity(n, k) > TKQ_RESCORE_CAP)
    return TKQ_ESHAPE;
  if (!aligned16(logits) || !aligned16(head) || !aligned16(x)) return TKQ_EALIGN;
  if ((reinterpret_cast<uintptr_t>(token) | reinterpret_cast<uintptr_t>(cand) |
       reinterpret_cast<uintptr_t>(cand_logits)) & 3u)
    return TKQ_EALIGN;
  return hip_status(tkq::launch_head_rescore(logits, n, head, x, K, k, token, cand, cand_logits,
                                             (hipStream_t)stream));
}

int tkq_gemv_argmax_rescore(const tkq_gemv_plan* plan, const tkq_gemv_desc* dev_descs, int32_t target, int64_t N,
                            int64_t K, const uint16_t* head, int32_t k, int32_t* token, int32_t* cand,
                            float* cand_logits, uint64_t* slots, int64_t scratch_bytes, void* stream) {
  const int st = check_plan(plan, dev_descs);
  if (st) return st;
  if (plan->fmt == TKQ_FMT_BIN) return TKQ_EFORMAT;
  if (target < 0 || target >= plan->count || !head || !token || !slots) return TKQ_EINVAL;
  if (scratch_bytes < 8 * plan->tiles || N < 1 || K < 1 || k < 1 || k > N) return TKQ_EINVAL;
  if (k > TKQ_RESCORE_MAX_K || N > INT32_MAX || K % 8 || K > TKQ_MAX_K ||
      tkq::rescore_capacity(N, k) > TKQ_RESCORE_CAP)
    return TKQ_ESHAPE;
  if (!aligned16(head) || !aligned16(slots)) return TKQ_EALIGN;
  if ((reinterpret_cast<uintptr_t>(token) | reinterpret_cast<uintptr_t>(cand) |
       reinterpret_cast<uintptr_t>(cand_logits)) & 3u)
    return TKQ_EALIGN;
  const hipError_t e = tkq::launch_gemv(plan->fmt, plan->variant, dev_descs, plan->count, plan->tiles, target,
                                        nullptr, slots, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(tkq::launch_gemv_rescore(dev_descs, plan->count, target, plan->tiles, slots, head, k, token,
                                             cand, cand_logits, (hipStream_t)stream));
}

int tkq_read_probe(const void* buf, int64_t bytes, uint32_t* out, void* stream) {
  if (!buf || !out || bytes < 16) return TKQ_EINVAL;
  if (bytes % 16) return TKQ_ESHAPE;
  if (!aligned16(buf) || !aligned16(out)) return TKQ_EALIGN;
  return hip_status(tkq::launch_read_probe(buf, bytes, out, (hipStream_t)stream));
}

}  // extern "C"

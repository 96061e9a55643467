// C ABI of libsmla.so: argument checks, the batch-sized split heuristic, workspace
// layout and kernel launches.  Declarations and contracts: include/smla.h.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "smla.h"
#include "smla_decode.hpp"
#include "smla_launch.hpp"

namespace {

using namespace smla;

constexpr int kMinTilesPerWg = 2;     // below this the partial results outweigh the rows
constexpr int kMinTilesPerSplit = 4;  // few tokens: tiles per split below which the merge outweighs them
constexpr int kMaxTopk = 65536;
constexpr uint64_t kMaxBufferBytes = 0xFFFFF000ull;   // byte range of one buffer resource (kOOB)

// Decode kernel for 16-head blocks, read once from SMLA_DECODE_VARIANT: "ring" (LDS-ring
// gather), "ws" (scoring and accumulating waves) or "regs" (register gather, PV overlapped
// with QK^T; the default).  Other head-block sizes have one kernel each.
int decode_variant() {
  static const int v = [] {
    const char* e = getenv("SMLA_DECODE_VARIANT");
    if (e != nullptr && strcmp(e, "ring") == 0) return 0;
    if (e != nullptr && strcmp(e, "ws") == 0) return 2;
    return 1;
  }();
  return v;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Workgroups per head block.  Few (token, head block) pairs: every token gets the same
// number of ranges, aligned to its tiles (so each range writes at most one partial and a
// token's merge reads few of them), one workgroup per CU.  Otherwise the stream-K ranges
// fill every resident workgroup slot once.
int32_t auto_splits(bool fp8rows, int32_t T, int32_t H, int32_t topk, bool grouped = false) {
  const int64_t cpt = (topk + kTileRows - 1) / kTileRows;
  const int64_t C = (int64_t)T * cpt;
  const int NG = heads_per_block_groups(H, topk, fp8rows, grouped);
  const int64_t HB = H / (kHeadGroup * NG);
  const int64_t cus = cu_count();
  int64_t G;
  if ((int64_t)T * HB < cus) {
    int64_t S = cus / ((int64_t)T * HB);
    const int64_t smax = cpt / kMinTilesPerSplit;
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    G = (int64_t)T * S;
  } else {
    G = cus * (grouped ? 1 : decode_wgs_per_cu(fp8rows, NG, decode_variant())) / HB;
    const int64_t cap = C / kMinTilesPerWg;
    if (G > cap) G = cap;
  }
  if (G < 1) G = 1;
  if (G > C) G = C;
  return (int32_t)G;
}

bool decode_shape_ok(int32_t T, int32_t H, int32_t topk) {
  return T >= 0 && H > 0 && topk >= 1 && topk <= kMaxTopk;
}

int check_decode(const void* q, const void* rows, int64_t pool_rows, const int32_t* idx, int32_t T,
                 int32_t H, int32_t topk, float softmax_scale, const void* out, const float* lse,
                 int32_t num_splits) {
  if (!decode_shape_ok(T, H, topk) || num_splits < 0 || pool_rows < 0 || !isfinite(softmax_scale) ||
      !(softmax_scale > 0.f))
    return SMLA_ERR_INVALID_ARG;
  if (H % kHeadGroup != 0) return SMLA_ERR_UNSUPPORTED;
  if (T == 0) return SMLA_OK;
  if (!q || !rows || !idx || !out || !lse) return SMLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(rows) || !aligned4(idx) || !aligned16(out) || !aligned4(lse))
    return SMLA_ERR_INVALID_ARG;
  return SMLA_OK;
}

// Scratch of sparse_mla_decode_noalloc (partials, their LSEs and the merge counters of
// the split work), one copy per GPU, held until the process ends.  Host code never uses
// this name as an address: scratch_address() looks up each device's copy.
static __device__ __align__(256) unsigned char scratch[SMLA_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device: hipGetSymbolAddress once per device,
// with that device current (each GPU holds its own copy at its own address); nullptr if the
// lookup fails.
void* scratch_address() {
  static std::atomic<void*> addr[64];
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = addr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

__global__ void zero_words_kernel(int32_t* p, int32_t n) {
  const int32_t i = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0;
}

// What `rows` holds: the NVFP4 pool, the staged FP8 rows of pass 2 (one per list entry),
// or a pool of FP8 rows.
enum class Rows { kNvfp4Pool, kFp8Staged, kFp8Pool };

// tok_heads > 0: grouped decode, with T groups of 64 heads made of the heads of
// 64 / tok_heads tokens, and union-list entries in idx.
int run_decode(Rows kind, const void* q, const void* rows, int64_t pool_rows,
               const int32_t* idx, int32_t T, int32_t H, int32_t topk, float softmax_scale,
               void* out, float* lse, int32_t num_splits, void* ws, size_t ws_bytes, void* stream,
               int32_t tok_heads = 0, const RowMap& map = identity_rowmap(), uint64_t alloc_rows = 0,
               bool clear_counters = false) {
  const bool grouped = tok_heads > 0;
  const bool fp8rows = kind != Rows::kNvfp4Pool;
  int st = check_decode(q, rows, pool_rows, idx, T, H, topk, softmax_scale, out, lse, num_splits);
  if (st != SMLA_OK || T == 0) return st;
  // every buffer the kernels address through a buffer resource must fit its byte range
  const uint64_t idx_bytes = (uint64_t)T * topk * 4;
  const uint64_t q_bytes = (uint64_t)T * H * 576 * 2;
  // (a block-major pool's allocation holds alloc_rows rows, every layer's)
  const uint64_t rows_bytes = kind == Rows::kFp8Staged ? (uint64_t)T * topk * 576
                              : alloc_rows > 0     ? alloc_rows * 352
                                                   : (uint64_t)pool_rows * (kind == Rows::kFp8Pool ? 576 : 352);
  if (idx_bytes > kMaxBufferBytes || rows_bytes > kMaxBufferBytes || q_bytes > kMaxBufferBytes)
    return SMLA_ERR_UNSUPPORTED;
  if ((int64_t)T * ((topk + kTileRows - 1) / kTileRows) >= (int64_t)1 << 31) return SMLA_ERR_UNSUPPORTED;
  const int32_t G = num_splits > 0 ? num_splits : auto_splits(fp8rows, T, H, topk, grouped);
  const DecodePlan p = make_plan(T, H, topk, G, fp8rows, grouped);
  if (p.bytes > kMaxBufferBytes) return SMLA_ERR_UNSUPPORTED;
  if (p.bytes > 0 && (ws == nullptr || ws_bytes < p.bytes || !aligned16(ws))) return SMLA_ERR_WORKSPACE;
  DecodeArgs a;
  a.q = q;
  a.rows = rows;
  a.pool_rows = pool_rows;
  a.idx = idx;
  a.T = T;
  a.H = H;
  a.topk = topk;
  a.cpt = p.cpt;
  a.tiles = p.tiles;
  a.G = p.G;
  a.HB = p.HB;
  a.rows_bytes = (uint32_t)rows_bytes;
  a.idx_bytes = (uint32_t)idx_bytes;
  a.q_bytes = (uint32_t)q_bytes;
  a.scale_log2 = softmax_scale * 1.44269504088896340736f;
  a.out = out;
  a.lse = lse;
  a.part_o = (float*)((char*)ws + p.part_o_off);
  a.part_lse = (float*)((char*)ws + p.part_lse_off);
  a.counters = (int32_t*)((char*)ws + p.counters_off);
  a.part_o_bytes = (uint32_t)(p.part_lse_off - p.part_o_off);
  a.part_lse_bytes = (uint32_t)(p.counters_off - p.part_lse_off);
  a.tok_heads = tok_heads;
  a.fp8_pool = kind == Rows::kFp8Pool;
  a.map = map;
  if (clear_counters) {   // a zero-fill kernel, not a memset node, so the call can be captured
    const int32_t n = p.HB * T;
    hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                       a.counters, n);
    if (hipGetLastError() != hipSuccess) return SMLA_ERR_LAUNCH;
  }
  const hipError_t e = grouped ? launch_decode_grouped(a, (hipStream_t)stream)
                       : fp8rows ? launch_decode_fp8rows(a, (hipStream_t)stream)
                                 : launch_decode_nvfp4(a, (hipStream_t)stream, decode_variant());
  return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

// Block-major multi-layer pool [pool_blocks][layers][block_rows][352]: the map of layer
// `layer`'s rows, or false for a malformed layout.  Block sizes are powers of two.
bool blhnc_map(int64_t pool_blocks, int32_t layers, int32_t layer, int32_t block_rows, RowMap& m) {
  if (pool_blocks < 0 || layers < 1 || layer < 0 || layer >= layers || block_rows < 1 ||
      block_rows > (1 << 16) || (block_rows & (block_rows - 1)) != 0)
    return false;
  uint32_t shift = 0;
  while ((1 << shift) < block_rows) shift++;
  m.shift = shift;
  m.mask = (uint32_t)block_rows - 1u;
  m.stride = (uint32_t)((int64_t)layers * block_rows);
  m.layer = (uint32_t)((int64_t)layer * block_rows);
  return (int64_t)layers * block_rows < (1 << 24);
}

// Grouped decode shapes: tpg tokens of H heads per group make the 64 heads of one block.
bool grouped_shape_ok(int32_t T, int32_t H, int32_t tpg, int32_t U) {
  return T >= 0 && H > 0 && tpg >= 1 && tpg <= kMaxGroupTokens && U >= 1 && U <= kMaxTopk &&
         T % tpg == 0;
}

}  // namespace

extern "C" {

SMLA_API const char* smla_status_string(int status) {
  switch (status) {
    case SMLA_OK: return "SMLA_OK";
    case SMLA_ERR_INVALID_ARG: return "SMLA_ERR_INVALID_ARG";
    case SMLA_ERR_UNSUPPORTED: return "SMLA_ERR_UNSUPPORTED";
    case SMLA_ERR_WORKSPACE: return "SMLA_ERR_WORKSPACE";
    case SMLA_ERR_LAUNCH: return "SMLA_ERR_LAUNCH";
    default: return "SMLA_ERR_UNKNOWN";
  }
}

SMLA_API int nvfp4_pack_rows(const void* src, const int32_t* slots, int32_t n, void* pool, int64_t pool_rows,
                    void* stream) {
  if (n < 0 || pool_rows < 0) return SMLA_ERR_INVALID_ARG;
  if (n == 0) return SMLA_OK;
  if (!src || !slots || !pool || !aligned16(src) || !aligned4(slots) || !aligned16(pool))
    return SMLA_ERR_INVALID_ARG;
  return launch_pack(src, slots, n, pool, pool_rows, identity_rowmap(), (hipStream_t)stream) == hipSuccess
             ? SMLA_OK
             : SMLA_ERR_LAUNCH;
}

SMLA_API int nvfp4_pack_rows_blhnc(const void* src, const int32_t* slots, int32_t n, void* pool,
                                   int64_t pool_blocks, int32_t layers, int32_t layer, int32_t block_rows,
                                   void* stream) {
  RowMap m;
  if (n < 0 || !blhnc_map(pool_blocks, layers, layer, block_rows, m)) return SMLA_ERR_INVALID_ARG;
  if (n == 0) return SMLA_OK;
  if (!src || !slots || !pool || !aligned16(src) || !aligned4(slots) || !aligned16(pool))
    return SMLA_ERR_INVALID_ARG;
  if (pool_blocks > ((int64_t)1 << 31) / block_rows) return SMLA_ERR_UNSUPPORTED;   // slots are int32
  return launch_pack(src, slots, n, pool, pool_blocks * block_rows, m, (hipStream_t)stream) == hipSuccess
             ? SMLA_OK
             : SMLA_ERR_LAUNCH;
}

SMLA_API int blhnc_copy_blocks(const void* src, int64_t src_blocks, const int32_t* src_ids, void* dst,
                               int64_t dst_blocks, const int32_t* dst_ids, int32_t n, int64_t block_bytes,
                               void* stream) {
  if (n < 0 || src_blocks < 0 || dst_blocks < 0 || block_bytes <= 0 || block_bytes % 16 != 0)
    return SMLA_ERR_INVALID_ARG;
  if (n == 0) return SMLA_OK;
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || (src_ids && !aligned4(src_ids)) ||
      (dst_ids && !aligned4(dst_ids)))
    return SMLA_ERR_INVALID_ARG;
  // segment ids are int32; the grid holds fewer than 2^24 workgroups of 256 lanes
  const uint64_t chunks = ((uint64_t)block_bytes / 16 + 1023) / 1024;
  if (block_bytes >= ((int64_t)1 << 36) || (uint64_t)n * chunks >= ((uint64_t)1 << 24))
    return SMLA_ERR_UNSUPPORTED;
  return launch_copy_segments(src, src_blocks, src_ids, dst, dst_blocks, dst_ids, n, block_bytes,
                              (hipStream_t)stream) == hipSuccess
             ? SMLA_OK
             : SMLA_ERR_LAUNCH;
}

SMLA_API int nvfp4_unpack_rows_f16(const void* pool, int64_t pool_rows, const int32_t* rows, int32_t n,
                          void* out, void* stream) {
  if (n < 0 || pool_rows < 0) return SMLA_ERR_INVALID_ARG;
  if (n == 0) return SMLA_OK;
  if (!pool || !rows || !out || !aligned16(pool) || !aligned4(rows) || !aligned16(out))
    return SMLA_ERR_INVALID_ARG;
  return launch_unpack(pool, pool_rows, rows, n, out, (hipStream_t)stream) == hipSuccess
             ? SMLA_OK
             : SMLA_ERR_LAUNCH;
}

SMLA_API int32_t smla_choose_num_splits(int32_t T, int32_t H, int32_t topk) {
  if (!decode_shape_ok(T, H, topk) || H % kHeadGroup != 0 || T == 0) return 0;
  return auto_splits(false, T, H, topk);
}

SMLA_API size_t smla_decode_workspace_bytes(int32_t T, int32_t H, int32_t topk, int32_t num_splits) {
  if (!decode_shape_ok(T, H, topk) || H % kHeadGroup != 0 || T == 0 || num_splits < 0) return 0;
  const int32_t G = num_splits > 0 ? num_splits : auto_splits(false, T, H, topk);
  const int32_t G8 = num_splits > 0 ? num_splits : auto_splits(true, T, H, topk);
  const size_t b4 = make_plan(T, H, topk, G, false).bytes, b8 = make_plan(T, H, topk, G8, true).bytes;
  return b4 > b8 ? b4 : b8;   // enough for either entry point
}

SMLA_API int sparse_mla_decode(const void* q, const void* pool, int64_t pool_rows, const int32_t* idx,
                      int32_t T, int32_t H, int32_t topk, float softmax_scale, void* out,
                      float* lse, int32_t num_splits, void* ws, size_t ws_bytes, void* stream) {
  return run_decode(Rows::kNvfp4Pool, q, pool, pool_rows, idx, T, H, topk, softmax_scale, out, lse,
                    num_splits, ws, ws_bytes, stream);
}

SMLA_API int sparse_mla_decode_noalloc(const void* q, const void* pool, int64_t pool_rows, const int32_t* idx,
                                       int32_t T, int32_t H, int32_t topk, float softmax_scale, void* out,
                                       float* lse, int32_t num_splits, void* stream) {
  // argument errors first, as in sparse_mla_decode, before the device lookup
  const int st = check_decode(q, pool, pool_rows, idx, T, H, topk, softmax_scale, out, lse, num_splits);
  if (st != SMLA_OK || T == 0) return st;
  void* ws = scratch_address();
  if (ws == nullptr) return SMLA_ERR_LAUNCH;
  return run_decode(Rows::kNvfp4Pool, q, pool, pool_rows, idx, T, H, topk, softmax_scale, out, lse,
                    num_splits, ws, SMLA_NOALLOC_SCRATCH_BYTES, stream, 0, identity_rowmap(), 0, true);
}

SMLA_API int sparse_mla_decode_blhnc(const void* q, const void* pool, int64_t pool_blocks, int32_t layers,
                                     int32_t layer, int32_t block_rows, const int32_t* idx, int32_t T,
                                     int32_t H, int32_t topk, float softmax_scale, void* out, float* lse,
                                     int32_t num_splits, void* ws, size_t ws_bytes, void* stream) {
  RowMap m;
  if (!blhnc_map(pool_blocks, layers, layer, block_rows, m)) return SMLA_ERR_INVALID_ARG;
  // layers * block_rows < 2^24 (checked above): bound the blocks first so the product cannot wrap
  if ((uint64_t)pool_blocks > kMaxBufferBytes / 352) return SMLA_ERR_UNSUPPORTED;
  const uint64_t alloc_rows = (uint64_t)pool_blocks * (uint64_t)layers * (uint64_t)block_rows;
  if (alloc_rows * 352 > kMaxBufferBytes) return SMLA_ERR_UNSUPPORTED;
  return run_decode(Rows::kNvfp4Pool, q, pool, pool_blocks * block_rows, idx, T, H, topk, softmax_scale,
                    out, lse, num_splits, ws, ws_bytes, stream, 0, m, alloc_rows);
}

SMLA_API int sparse_mla_combine(const float* part_o, const float* part_lse, int32_t T, int32_t S, int32_t H,
                       void* out, float* lse, void* stream) {
  if (T < 0 || S < 1 || H <= 0) return SMLA_ERR_INVALID_ARG;
  if (H % kHeadGroup != 0) return SMLA_ERR_UNSUPPORTED;
  if (T == 0) return SMLA_OK;
  if (!part_o || !part_lse || !out || !lse || !aligned16(part_o) || !aligned4(part_lse) ||
      !aligned16(out) || !aligned4(lse))
    return SMLA_ERR_INVALID_ARG;
  if ((uint64_t)T * S * H * 512 * 4 > kMaxBufferBytes) return SMLA_ERR_UNSUPPORTED;
  return launch_combine(part_o, part_lse, T, S, H, out, lse, (hipStream_t)stream) == hipSuccess
             ? SMLA_OK
             : SMLA_ERR_LAUNCH;
}

SMLA_API int nvfp4_stage_fp8(const void* pool, int64_t pool_rows, const int32_t* idx, int32_t T, int32_t topk,
                    void* staged, void* stream) {
  if (T < 0 || topk < 1 || topk > kMaxTopk || pool_rows < 0) return SMLA_ERR_INVALID_ARG;
  if (T == 0) return SMLA_OK;
  if (!pool || !idx || !staged || !aligned16(pool) || !aligned4(idx) || !aligned16(staged))
    return SMLA_ERR_INVALID_ARG;
  return launch_stage_fp8(pool, pool_rows, idx, (int64_t)T * topk, staged, (hipStream_t)stream) ==
                 hipSuccess
             ? SMLA_OK
             : SMLA_ERR_LAUNCH;
}

SMLA_API int sparse_mla_decode_fp8rows(const void* q, const void* staged, const int32_t* idx,
                              int64_t pool_rows, int32_t T, int32_t H, int32_t topk,
                              float softmax_scale, void* out, float* lse, int32_t num_splits,
                              void* ws, size_t ws_bytes, void* stream) {
  return run_decode(Rows::kFp8Staged, q, staged, pool_rows, idx, T, H, topk, softmax_scale, out, lse,
                    num_splits, ws, ws_bytes, stream);
}

SMLA_API int fp8_pack_rows(const void* src, const int32_t* slots, int32_t n, void* pool, int64_t pool_rows,
                           void* stream) {
  if (n < 0 || pool_rows < 0) return SMLA_ERR_INVALID_ARG;
  if (n == 0) return SMLA_OK;
  if (!src || !slots || !pool || !aligned16(src) || !aligned4(slots) || !aligned16(pool))
    return SMLA_ERR_INVALID_ARG;
  return launch_fp8_pack(src, slots, n, pool, pool_rows, (hipStream_t)stream) == hipSuccess ? SMLA_OK
                                                                                            : SMLA_ERR_LAUNCH;
}

SMLA_API int sparse_mla_decode_fp8pool(const void* q, const void* pool, int64_t pool_rows, const int32_t* idx,
                                       int32_t T, int32_t H, int32_t topk, float softmax_scale, void* out,
                                       float* lse, int32_t num_splits, void* ws, size_t ws_bytes,
                                       void* stream) {
  return run_decode(Rows::kFp8Pool, q, pool, pool_rows, idx, T, H, topk, softmax_scale, out, lse,
                    num_splits, ws, ws_bytes, stream);
}

SMLA_API int smla_group_union(const int32_t* idx, int32_t T, int32_t topk, int32_t tpg, int64_t pool_rows,
                              int32_t U, int32_t* uni, int32_t* count, void* stream) {
  if (T < 0 || tpg < 1 || tpg > kMaxGroupTokens || topk < 1 || U < 1 || pool_rows < 0 || T % tpg != 0)
    return SMLA_ERR_INVALID_ARG;
  if ((int64_t)tpg * topk > kMaxGroupEntries || pool_rows > (int64_t)kRowMask + 1) return SMLA_ERR_UNSUPPORTED;
  if (T == 0) return SMLA_OK;
  if (!idx || !uni || !count || !aligned4(idx) || !aligned4(uni) || !aligned4(count)) return SMLA_ERR_INVALID_ARG;
  return launch_group_union(idx, T, topk, tpg, pool_rows, U, uni, count, (hipStream_t)stream) == hipSuccess
             ? SMLA_OK
             : SMLA_ERR_LAUNCH;
}

SMLA_API size_t smla_decode_grouped_workspace_bytes(int32_t T, int32_t H, int32_t tpg, int32_t U,
                                                    int32_t num_splits) {
  if (!grouped_shape_ok(T, H, tpg, U) || (int64_t)H * tpg != 4 * kHeadGroup || T == 0 || num_splits < 0) return 0;
  const int32_t G = num_splits > 0 ? num_splits : auto_splits(false, T / tpg, 4 * kHeadGroup, U, true);
  return make_plan(T / tpg, 4 * kHeadGroup, U, G, false, true).bytes;
}

SMLA_API int sparse_mla_decode_grouped(const void* q, const void* pool, int64_t pool_rows, const int32_t* uni,
                                       int32_t T, int32_t H, int32_t tpg, int32_t U, float softmax_scale,
                                       void* out, float* lse, int32_t num_splits, void* ws, size_t ws_bytes,
                                       void* stream) {
  if (!grouped_shape_ok(T, H, tpg, U)) return SMLA_ERR_INVALID_ARG;
  if ((int64_t)H * tpg != 4 * kHeadGroup || pool_rows > (int64_t)kRowMask + 1) return SMLA_ERR_UNSUPPORTED;
  return run_decode(Rows::kNvfp4Pool, q, pool, pool_rows, uni, T / tpg, 4 * kHeadGroup, U, softmax_scale, out,
                    lse, num_splits, ws, ws_bytes, stream, H);
}

}  // extern "C"

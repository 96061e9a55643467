// Work decomposition of the sparse MLA decode shared by the host API and the kernels.
//
// "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section
// "Four-bit caches make room": the native kernel sizes its parallel decomposition by the
// token batch.  Here every token's index list is cut into tiles of kTileRows entries; the
// T*ceil(topk/kTileRows) tiles form one flat sequence that G workgroups per head block
// split into equal contiguous ranges (a stream-K split over the index lists).  A range
// that covers all of a token's tiles writes that token's output directly; a token shared
// by several ranges gets one normalized partial result from each, and the range that
// finishes last merges them with a log-sum-exp combine in the same launch.  A range
// shares at most two tokens with other ranges (its first and its last), so each
// workgroup owns two partial slots.
//
// Heads are processed in blocks of 16*NG: one workgroup gathers and unpacks a row once
// and applies it to all heads of its block.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace smla {

constexpr int kTileRows = 64;    // index-list entries per tile
constexpr int kHeadGroup = 16;   // heads per MFMA tile

// Grouped decode (the tokens of a session share most of their list entries): each group of
// up to kMaxGroupTokens consecutive tokens attends over one union list whose entries are
// row | (members << kMemberShift); bit i of members says that token i of the group lists
// the row.  A negative entry is empty.
constexpr int kMemberShift = 27;
constexpr int32_t kRowMask = (1 << kMemberShift) - 1;
constexpr int kMaxGroupTokens = 4;
constexpr int kMaxGroupEntries = 8192;   // tokens per group x topk the union builder takes

// Where row v of a layer's list lives in the allocation the kernels read.  A layer-major
// pool holds the layer's rows one after another (identity map).  A block-major
// multi-layer pool ("Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily",
// section on the BLHNC layout: the data of several layers stored together for each block)
// is [block][layer][row in block][row bytes], so row v of layer l sits at allocation row
// ((v >> shift) * stride + layer) + (v & mask), with block size B = 1 << shift,
// mask = B - 1, stride = layers * B and layer = l * B.
struct RowMap {
  uint32_t shift, mask, stride, layer;
};
__host__ __device__ inline RowMap identity_rowmap() { return RowMap{0u, 0u, 1u, 0u}; }
// Every term stays below 2^24 (the host bounds the allocation by the buffer range, which
// holds fewer than 2^24 rows), so the 24-bit multiply is exact.
__device__ __forceinline__ uint32_t storage_row(uint32_t v, const RowMap& m) {
  return __umul24(v >> m.shift, m.stride) + m.layer + (v & m.mask);
}
// The same for any non-negative row id, in 64 bits (writers, whose pools are not bounded).
__host__ __device__ inline uint64_t storage_row_wide(uint32_t v, const RowMap& m) {
  return (uint64_t)(v >> m.shift) * m.stride + m.layer + (v & m.mask);
}

struct DecodeArgs {
  const void* q;            // fp16 [T][H][576]
  const void* rows;         // NVFP4 pool [pool_rows][352], staged FP8 rows [T*topk][576],
                            // or (fp8_pool) an FP8 pool [pool_rows][576]
  int64_t pool_rows;
  const int32_t* idx;       // [T][topk]
  int32_t T, H, topk;
  int32_t cpt;              // tiles per token = ceil(topk / kTileRows)
  int64_t tiles;            // T * cpt
  int32_t G;                // ranges (workgroups) per head block
  int32_t HB;               // head blocks = H / (16 * NG)
  uint32_t rows_bytes;      // bytes addressable through `rows`
  uint32_t idx_bytes;       // bytes of `idx`
  uint32_t q_bytes;         // bytes of `q`
  float scale_log2;         // softmax_scale * log2(e)
  void* out;                // fp16 [T][H][512]
  float* lse;               // fp32 [T][H]
  float* part_o;            // fp32 [HB][G][2][16*NG][512]
  float* part_lse;          // fp32 [HB][G][2][16*NG]
  int32_t* counters;        // [HB][T], zero between launches
  int32_t tok_heads;        // grouped decode: heads per real token (entries carry membership bits); else 0
  uint32_t part_o_bytes;    // bytes of part_o
  uint32_t part_lse_bytes;  // bytes of part_lse
  int32_t fp8_pool;         // FP8 rows: 1 = row v of a pool, 0 = the staged row of entry (t, j)
  RowMap map;               // list row -> allocation row of a pool (identity unless block-major)
};

struct DecodePlan {
  int32_t cpt, G, HB, NG;
  int64_t tiles;
  size_t part_o_off, part_lse_off, counters_off, bytes;
};

// First tile of range w: floor(w * C / G).
__host__ __device__ inline int64_t wg_first_chunk(int64_t w, int64_t C, int64_t G) {
  return w * C / G;
}
// The range that holds tile c: the largest w with floor(w*C/G) <= c.
__host__ __device__ inline int64_t wg_of_chunk(int64_t c, int64_t C, int64_t G) {
  return ((c + 1) * G - 1) / C;
}

// Head groups of 16 per workgroup.  The unpack of a row is shared by all heads of a block,
// so blocks are as large as the head count allows: 64 heads (NVFP4 rows only), else 32,
// else 16.  Blocks of 32 or 64 need a token to span at least two tiles (those kernels
// stage one query at a time).  Grouped decode always runs 64-head blocks (the heads of
// the tokens of one group).
inline int32_t heads_per_block_groups(int32_t H, int32_t topk, bool fp8rows, bool grouped = false) {
  if (grouped) return 4;
  if (topk <= kTileRows) return 1;
  if (H % (4 * kHeadGroup) == 0) return 4;
  return H % (2 * kHeadGroup) == 0 ? 2 : 1;
}

inline DecodePlan make_plan(int32_t T, int32_t H, int32_t topk, int32_t G, bool fp8rows, bool grouped = false) {
  DecodePlan p;
  p.cpt = (topk + kTileRows - 1) / kTileRows;
  p.tiles = (int64_t)T * p.cpt;
  p.NG = heads_per_block_groups(H, topk, fp8rows, grouped);
  p.HB = H / (kHeadGroup * p.NG);
  if (G > p.tiles) G = (int32_t)p.tiles;
  if (G < 1) G = 1;
  p.G = G;
  const size_t slots = (size_t)p.HB * p.G * 2;
  const size_t heads = (size_t)kHeadGroup * p.NG;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.part_o_off = 0;
  p.part_lse_off = up(slots * heads * 512 * sizeof(float));
  p.counters_off = p.part_lse_off + up(slots * heads * sizeof(float));
  p.bytes = p.counters_off + up((size_t)p.HB * T * sizeof(int32_t));
  return p;
}

}  // namespace smla

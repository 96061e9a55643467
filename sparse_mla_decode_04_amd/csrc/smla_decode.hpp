// Work decomposition of the sparse MLA decode shared by the host API and the kernels.
//
// "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section
// "Four-bit caches make room": the native kernel sizes its parallel decomposition by the
// token batch.  Here the T index lists are cut into chunks of kChunkRows entries; the
// T*ceil(topk/kChunkRows) chunks of every 16-head group form one flat sequence that G
// workgroups split into equal contiguous ranges (a stream-K split over the index lists).
// A workgroup whose range covers a token's chunks entirely writes the final output; the
// workgroups that share a token write normalized partial results, and the last of them
// to finish merges those partials with a log-sum-exp combine in the same launch.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace smla {

constexpr int kChunkRows = 64;   // list entries per chunk
constexpr int kHeadGroup = 16;   // heads per workgroup (MFMA N / M dimension)

struct DecodeArgs {
  const void* q;            // fp16 [T][H][576]
  const void* rows;         // NVFP4 pool [pool_rows][352], or staged FP8 rows [T*topk][576]
  int64_t pool_rows;
  const int32_t* idx;       // [T][topk]
  int32_t T, H, topk;
  int32_t cpt;              // chunks per token = ceil(topk / kChunkRows)
  int64_t chunks;           // T * cpt
  int32_t G;                // workgroups per head group
  int32_t max_seg;          // partial slots per workgroup
  float scale_log2;         // softmax_scale * log2(e)
  void* out;                // fp16 [T][H][512]
  float* lse;               // fp32 [T][H]
  float* part_o;            // fp32 [HG][G][max_seg][16][512]
  float* part_lse;          // fp32 [HG][G][max_seg][16]
  int32_t* counters;        // [HG][T]
};

struct DecodePlan {
  int32_t cpt, G, max_seg, HG;
  int64_t chunks;
  size_t part_o_off, part_lse_off, counters_off, bytes;
};

// First chunk of workgroup w: floor(w * C / G).
__host__ __device__ inline int64_t wg_first_chunk(int64_t w, int64_t C, int64_t G) {
  return w * C / G;
}
// The workgroup whose range holds chunk c: the largest w with floor(w*C/G) <= c.
__host__ __device__ inline int64_t wg_of_chunk(int64_t c, int64_t C, int64_t G) {
  return ((c + 1) * G - 1) / C;
}

inline DecodePlan make_plan(int32_t T, int32_t H, int32_t topk, int32_t G) {
  DecodePlan p;
  p.cpt = (topk + kChunkRows - 1) / kChunkRows;
  p.chunks = (int64_t)T * p.cpt;
  p.HG = H / kHeadGroup;
  if (G > p.chunks) G = (int32_t)p.chunks;
  if (G < 1) G = 1;
  p.G = G;
  const int64_t per_wg = (p.chunks + G - 1) / G;          // most chunks one workgroup gets
  p.max_seg = (int32_t)((per_wg + p.cpt - 1) / p.cpt + 1);  // tokens one workgroup can touch
  const size_t slots = (size_t)p.HG * p.G * p.max_seg;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.part_o_off = 0;
  p.part_lse_off = up(slots * kHeadGroup * 512 * sizeof(float));
  p.counters_off = p.part_lse_off + up(slots * kHeadGroup * sizeof(float));
  p.bytes = p.counters_off + up((size_t)p.HG * T * sizeof(int32_t));
  return p;
}

}  // namespace smla

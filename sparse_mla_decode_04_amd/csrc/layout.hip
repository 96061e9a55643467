// Block transfers of a block-major multi-layer cache for gfx950.
//
// "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section on the
// BLHNC layout: storing the data of several layers together for each block makes one
// block of every layer a single contiguous piece, so moving a request's cache takes one
// transfer per block instead of one per block and layer.  On one GPU the transfer is the
// gather of a request's blocks into a contiguous send buffer (and the scatter of a
// received buffer into free blocks): a copy of whole segments, bound by HBM.
#include "smla_device.hpp"
#include "smla_launch.hpp"

namespace smla {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;                                   // 16-byte pieces per thread
constexpr uint32_t kCopyChunk = kCopyThreads * kCopyUnroll;      // pieces per workgroup

// Workgroup w copies chunk w % chunks of segment w / chunks: up to kCopyChunk 16-byte
// pieces, every load of a thread issued before its stores.  A segment whose source or
// destination id is outside its array is skipped (a wave-uniform test).  The data is not
// read again by this launch, so the loads and stores are non-temporal.
__global__ __launch_bounds__(kCopyThreads) void copy_segments_kernel(
    const uint8_t* __restrict__ src, int64_t src_segs, const int32_t* __restrict__ src_ids,
    uint8_t* __restrict__ dst, int64_t dst_segs, const int32_t* __restrict__ dst_ids, uint32_t chunks,
    uint32_t pieces, int64_t seg_bytes) {
  const uint32_t seg = blockIdx.x / chunks, chunk = blockIdx.x - seg * chunks;
  const int64_t s = src_ids ? (int64_t)src_ids[seg] : (int64_t)seg;
  const int64_t d = dst_ids ? (int64_t)dst_ids[seg] : (int64_t)seg;
  if (s < 0 || s >= src_segs || d < 0 || d >= dst_segs) return;
  const u32x4* sp = (const u32x4*)(src + s * seg_bytes);
  u32x4* dp = (u32x4*)(dst + d * seg_bytes);
  const uint32_t p0 = chunk * kCopyChunk + threadIdx.x;
  u32x4 v[kCopyUnroll];
#pragma unroll
  for (int k = 0; k < kCopyUnroll; k++) {
    const uint32_t p = p0 + k * kCopyThreads;
    if (p < pieces) v[k] = __builtin_nontemporal_load(sp + p);
  }
#pragma unroll
  for (int k = 0; k < kCopyUnroll; k++) {
    const uint32_t p = p0 + k * kCopyThreads;
    if (p < pieces) __builtin_nontemporal_store(v[k], dp + p);
  }
}

hipError_t launch_copy_segments(const void* src, int64_t src_segs, const int32_t* src_ids, void* dst,
                                int64_t dst_segs, const int32_t* dst_ids, int32_t n, int64_t seg_bytes,
                                hipStream_t s) {
  const uint32_t pieces = (uint32_t)(seg_bytes / 16);
  const uint32_t chunks = (pieces + kCopyChunk - 1) / kCopyChunk;
  hipLaunchKernelGGL(copy_segments_kernel, dim3((uint32_t)n * chunks), dim3(kCopyThreads), 0, s,
                     (const uint8_t*)src, src_segs, src_ids, (uint8_t*)dst, dst_segs, dst_ids, chunks,
                     pieces, seg_bytes);
  return hipGetLastError();
}

}  // namespace smla

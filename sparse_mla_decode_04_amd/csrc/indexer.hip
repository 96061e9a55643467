// Top-k selection of the sparse indexer (gfx950 / MI355X), and its C entry point.
//
// "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section "Four-bit
// caches make room": a sparse indexer picks 2,048 context positions per decode token, and
// the decode kernel loads only their cache rows.  The page gives no internals of the
// indexer's scoring (trained weights); this is the step that turns given float32 scores
// into the index list:
//   * token t has lengths[t] positions 0 .. lengths[t] - 1; its list holds the k positions
//     with the largest scores, equal scores (as numbers, -0 == +0) going to the lower
//     position;
//   * entries are row_offset[t] + position, in ascending position order; a token with fewer
//     than k positions lists them all, then -1.
//
// One workgroup per token: 1,024 threads when the tokens fit the CUs once, else 512.  With
// at most half as many tokens as CUs, each token's positions are split over several
// workgroups instead (indexer_split.hpp), given a workspace.
// Scores map to 32-bit keys whose unsigned order is the numbers' order; the k-th largest
// key K is found by a radix select over 11, 11 and 10 key bits (each step histograms, in
// LDS, the keys that share the bits chosen so far; a prefix sum over the bins from the top
// picks the bin holding the k-th key).
//   pass 1 (HBM): histogram of the top 11 bits of every key -> the bin b of the k-th key.
//   pass 2 (L2):  keys above bin b are in the list: their positions are set in an LDS
//                 bitmap; keys in bin b go to LDS with their positions (with N(0,1)-like
//                 scores a few thousand).
//   in LDS:       the two remaining radix steps over bin b's keys give K and how many keys
//                 equal to K the list takes (`need`, lowest positions first); bin b's keys
//                 above K join the bitmap, those equal to K go to a second one; popcount
//                 prefix sums over the bitmap words then write the list in position order.
// A context longer than the bitmaps, or a cut bin with more keys than LDS keeps (for
// instance nearly equal scores), takes the remaining radix steps and the ordered write
// from the scores in memory instead.
#include <hip/hip_runtime.h>

#include <atomic>

#include "smla.h"

namespace {

// Few tokens (at most one workgroup per CU): 1,024 threads per token hide more latency.
// More tokens: 512 threads, so that two workgroups share a CU.
namespace wg1024 {
constexpr int kThreadsK = 1024;
#include "indexer_body.hpp"
#include "indexer_split.hpp"
}  // namespace wg1024
namespace wg512 {
constexpr int kThreadsK = 512;
#include "indexer_body.hpp"
}  // namespace wg512

int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool aligned_to(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

constexpr int kMaxParts = 64;        // workgroups per token of the split selection
constexpr int64_t kMinChunk = 8192;  // positions per workgroup the automatic split keeps at least

// Workgroups per token: `parts` when given, else a split that fills the CUs once when the
// tokens fill at most half of them (each chunk keeping kMinChunk positions), else 1.
int32_t indexer_parts(int32_t T, int64_t ld, int32_t parts) {
  if (parts > 0) return parts;
  const int cus = device_cus();
  if (T < 1 || 2 * (int64_t)T > cus) return 1;
  int64_t P = cus / T;
  if (P > kMaxParts) P = kMaxParts;
  if (P > ld / kMinChunk) P = ld / kMinChunk;
  return P >= 2 ? (int32_t)P : 1;
}

bool indexer_args_ok(int32_t T, int64_t ld, int32_t k, int32_t parts) {
  return T >= 0 && k >= 1 && k <= wg512::kMaxK && ld >= 0 && ld % 4 == 0 && ld <= INT32_MAX && parts >= 0 &&
         parts <= kMaxParts;
}

}  // namespace

extern "C" SMLA_API size_t smla_indexer_workspace_bytes(int32_t T, int64_t ld, int32_t k, int32_t parts) {
  if (!indexer_args_ok(T, ld, k, parts) || T == 0) return 0;
  const int32_t P = indexer_parts(T, ld, parts);
  if (P < 2 || T > 65535) return 0;
  return wg1024::split_ws_layout(T, P, nullptr, nullptr);
}

extern "C" SMLA_API int sparse_indexer_topk(const float* scores, int64_t ld, const int32_t* lengths,
                                            const int32_t* row_offset, int32_t T, int32_t k, int32_t* out,
                                            int32_t parts, void* ws, size_t ws_bytes, void* stream) {
  if (!indexer_args_ok(T, ld, k, parts)) return SMLA_ERR_INVALID_ARG;
  if (T == 0) return SMLA_OK;
  if (!out || !aligned_to(out, 4) || (ld > 0 && (!scores || !aligned_to(scores, 16))) ||
      (lengths && !aligned_to(lengths, 4)) || (row_offset && !aligned_to(row_offset, 4)))
    return SMLA_ERR_INVALID_ARG;
  const int32_t P = indexer_parts(T, ld, parts);
  if (P >= 2 && T > 65535) return SMLA_ERR_UNSUPPORTED;   // the split launches put tokens on grid y
  if (P >= 2 && ws != nullptr) {
    if (!aligned_to(ws, 16) || ws_bytes < wg1024::split_ws_layout(T, P, nullptr, nullptr)) return SMLA_ERR_WORKSPACE;
    wg1024::SplitWs v;
    wg1024::split_ws_layout(T, P, ws, &v);
    const hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(wg1024::topk_split_hist_kernel, dim3(P, T), dim3(wg1024::kThreadsK), 0, s, scores, ld,
                       lengths, k, P, v);
    hipLaunchKernelGGL(wg1024::topk_split_classify_kernel, dim3(P, T), dim3(wg1024::kThreadsK), 0, s, scores, ld,
                       lengths, row_offset, k, P, out, v);
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
  }
  if (parts >= 2) return SMLA_ERR_WORKSPACE;   // a split asked for without a workspace
  if (T <= device_cus())
    hipLaunchKernelGGL(wg1024::sparse_indexer_topk_kernel, dim3(T), dim3(wg1024::kThreadsK), 0, (hipStream_t)stream,
                       scores, ld, lengths, row_offset, k, out);
  else
    hipLaunchKernelGGL(wg512::sparse_indexer_topk_kernel, dim3(T), dim3(wg512::kThreadsK), 0, (hipStream_t)stream,
                       scores, ld, lengths, row_offset, k, out);
  return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

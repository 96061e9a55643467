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
// One workgroup of 1,024 threads per token.  Scores map to 32-bit keys whose unsigned order
// is the numbers' order.  A radix select finds the k-th largest key K in three passes over
// the token's scores (11, 11 and 10 key bits; each pass histograms, in LDS, the keys that
// share the bits chosen so far, and a prefix sum over the bins from the top picks the bin
// that holds the k-th key).  A last pass writes, in position order, every key above K and
// the first `need` keys equal to K, placing each by a workgroup prefix sum of the counts.
// The first pass reads the scores from HBM; the later ones mostly hit L2 / the Infinity
// Cache (a 140,000-position token is 560 KB).
#include <hip/hip_runtime.h>

#include "smla.h"

namespace {

constexpr int kThreadsK = 1024;
constexpr int kWavesK = kThreadsK / 64;
constexpr int kBins = 2048;
constexpr int kMaxK = 65536;

struct SmemTopk {
  uint32_t hist[kBins];
  uint32_t wsum[kWavesK];
  uint32_t pick[2];   // chosen bin, keys above it
};

// Unsigned order of the key = numeric order of the score; -0 maps to the key of +0.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum of v over the workgroup's threads in thread order; `total` gets the
// sum over all threads.  Every thread must call it.
__device__ __forceinline__ uint32_t block_scan(SmemTopk& sm, uint32_t v, uint32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sm.wsum[w] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWavesK; i++) {
    const uint32_t s = sm.wsum[i];
    before += i < w ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return x + before;
}

// Keys of positions p0 .. p0 + 3 (those below n); `in` marks which exist.
__device__ __forceinline__ void load_keys(const float* __restrict__ s, int64_t p0, int64_t n, uint32_t (&key)[4],
                                          bool (&in)[4]) {
  if (p0 + 3 < n) {
    const float4 v = *(const float4*)(s + p0);
    key[0] = score_key(v.x);
    key[1] = score_key(v.y);
    key[2] = score_key(v.z);
    key[3] = score_key(v.w);
    in[0] = in[1] = in[2] = in[3] = true;
  } else {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      in[j] = p0 + j < n;
      key[j] = in[j] ? score_key(s[p0 + j]) : 0u;
    }
  }
}

__global__ __launch_bounds__(kThreadsK) void sparse_indexer_topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                                       const int32_t* __restrict__ lengths,
                                                                       const int32_t* __restrict__ row_offset,
                                                                       int32_t k, int32_t* __restrict__ out) {
  __shared__ SmemTopk sm;
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  int64_t n = lengths ? (int64_t)lengths[t] : ld;
  n = n < 0 ? 0 : (n > ld ? ld : n);
  const int32_t off = row_offset ? row_offset[t] : 0;
  const float* s = scores + t * ld;
  int32_t* o = out + t * (int64_t)k;
  if (n <= k) {   // every position, then empties
    for (int p = tid; p < k; p += kThreadsK) o[p] = p < n ? off + p : -1;
    return;
  }

  // ---- radix select: after the passes, prefix = K (the k-th largest key) and `need` keys
  // equal to K belong to the list (the count of keys equal to K is at least need >= 1)
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
  for (int pass = 0; pass < 3; pass++) {
    const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    const uint32_t bmask = pass == 2 ? 1023u : 2047u;
    for (int i = tid; i < kBins; i += kThreadsK) sm.hist[i] = 0;
    __syncthreads();
    for (int64_t p0 = 4 * tid; p0 < n; p0 += 4 * kThreadsK) {
      uint32_t key[4];
      bool in[4];
      load_keys(s, p0, n, key, in);
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (in[j] && (key[j] & pmask) == prefix) atomicAdd(&sm.hist[(key[j] >> shift) & bmask], 1u);
    }
    __syncthreads();
    // thread tid holds the bins of descending rank 2 tid and 2 tid + 1
    const int b0 = (int)bmask - 2 * tid, b1 = b0 - 1;
    const uint32_t h0 = b0 >= 0 ? sm.hist[b0] : 0u, h1 = b1 >= 0 ? sm.hist[b1] : 0u;
    uint32_t tot;
    const uint32_t before = block_scan(sm, h0 + h1, tot) - h0 - h1;   // keys in higher bins
    if (before < need && need <= before + h0) {
      sm.pick[0] = (uint32_t)b0;
      sm.pick[1] = before;
    } else if (before + h0 < need && need <= before + h0 + h1) {
      sm.pick[0] = (uint32_t)b1;
      sm.pick[1] = before + h0;
    }
    __syncthreads();
    prefix |= sm.pick[0] << shift;
    pmask |= bmask << shift;
    need -= sm.pick[1];
    __syncthreads();
  }
  const uint32_t K = prefix;

  // ---- write the list in position order: keys above K, and the first `need` keys equal to
  // K.  gb / eb: keys above K / equal to K at lower positions; an entry goes to gb +
  // min(eb, need).
  uint32_t gt_run = 0, eq_run = 0;
  for (int64_t c = 0; c < n; c += 4 * kThreadsK) {
    const int64_t p0 = c + 4 * tid;
    uint32_t key[4];
    bool in[4];
    load_keys(s, p0, n, key, in);
    uint32_t g = 0, e = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      g += (in[j] && key[j] > K) ? 1u : 0u;
      e += (in[j] && key[j] == K) ? 1u : 0u;
    }
    const uint32_t mine = g | (e << 16);   // at most 4,096 of each per chunk
    uint32_t tot;
    const uint32_t excl = block_scan(sm, mine, tot) - mine;
    uint32_t gb = gt_run + (excl & 0xFFFFu), eb = eq_run + (excl >> 16);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (!in[j]) continue;
      const int32_t entry = off + (int32_t)(p0 + j);
      // the places are below k by construction; the test only keeps a write inside the row
      if (key[j] > K) {
        const uint32_t at = gb + (eb < need ? eb : need);
        if (at < (uint32_t)k) o[at] = entry;
        gb++;
      } else if (key[j] == K) {
        if (eb < need && gb + eb < (uint32_t)k) o[gb + eb] = entry;
        eb++;
      }
    }
    gt_run += tot & 0xFFFFu;
    eq_run += tot >> 16;
  }
}

bool aligned_to(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace

extern "C" SMLA_API int sparse_indexer_topk(const float* scores, int64_t ld, const int32_t* lengths,
                                            const int32_t* row_offset, int32_t T, int32_t k, int32_t* out,
                                            void* stream) {
  if (T < 0 || k < 1 || k > kMaxK || ld < 0 || ld % 4 != 0 || ld > INT32_MAX) return SMLA_ERR_INVALID_ARG;
  if (T == 0) return SMLA_OK;
  if (!out || !aligned_to(out, 4) || (ld > 0 && (!scores || !aligned_to(scores, 16))) ||
      (lengths && !aligned_to(lengths, 4)) || (row_offset && !aligned_to(row_offset, 4)))
    return SMLA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(sparse_indexer_topk_kernel, dim3(T), dim3(kThreadsK), 0, (hipStream_t)stream, scores, ld,
                     lengths, row_offset, k, out);
  return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

// Top-k selection split over several workgroups per token (see indexer.hip), included after
// indexer_body.hpp in the namespace of one workgroup size.
//
// One workgroup per token leaves most CUs idle when there are few tokens.  Here token t's
// positions are cut into P chunks (whole bitmap words each) and two launches do the work:
//   hist:     workgroup (c, t) histograms the top 11 key bits of chunk c into memory; the
//             last of the token's P workgroups (a device-scope counter) adds the P
//             histograms and picks the bin of the k-th key -> rec[t] = {bin, need}.
//   classify: workgroup (c, t) reads chunk c again: keys above the bin become bits of the
//             token's bitmap in memory, keys in the bin go with their positions to the
//             token's cut buffer (one reservation per workgroup).  The last of the token's
//             workgroups loads bitmap and cut keys into LDS and finishes as the
//             single-workgroup kernel does, or from the scores in memory when the context is
//             longer than the bitmap or the cut bin holds more keys than LDS keeps.
// The result is the single-workgroup kernel's, bit for bit: the same histograms, the same K,
// the same ordered write.

static_assert(kCap % kThreadsK == 0, "every thread loads the same number of cut keys");

// Views into the workspace (zero before the first call; every call leaves it zero where it
// must start at zero: the arrival counters and the cut counts).
struct SplitWs {
  uint32_t* hist;    // [T][P][kBins] chunk histograms
  int32_t* arrive;   // [T] workgroups of the token done with the histogram
  uint32_t* rec;     // [T][2] bin of the k-th key, keys of the list from that bin on
  uint32_t* bmap;    // [T][kMapWords] keys above the bin
  int32_t* ccount;   // [T] keys of the bin
  uint32_t* ckey;    // [T][kCap] keys of the bin
  int32_t* cpos;     // [T][kCap] their positions
};

inline size_t split_ws_layout(int64_t T, int64_t P, void* base, SplitWs* v) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t o = 0;
  const size_t hist = o;
  o += up((size_t)T * P * kBins * 4);
  const size_t arrive = o;
  o += up((size_t)T * 4);
  const size_t rec = o;
  o += up((size_t)T * 8);
  const size_t bmap = o;
  o += up((size_t)T * kMapWords * 4);
  const size_t ccount = o;
  o += up((size_t)T * 4);
  const size_t ckey = o;
  o += up((size_t)T * kCap * 4);
  const size_t cpos = o;
  o += up((size_t)T * kCap * 4);
  if (v != nullptr) {
    char* b = (char*)base;
    v->hist = (uint32_t*)(b + hist);
    v->arrive = (int32_t*)(b + arrive);
    v->rec = (uint32_t*)(b + rec);
    v->bmap = (uint32_t*)(b + bmap);
    v->ccount = (int32_t*)(b + ccount);
    v->ckey = (uint32_t*)(b + ckey);
    v->cpos = (int32_t*)(b + cpos);
  }
  return o;
}

// Chunk c of a token of n positions: [lo, hi), lo a multiple of 32 (chunks own whole bitmap
// words and start 16-byte aligned).
__device__ __forceinline__ void split_chunk(int64_t n, int32_t P, int32_t c, int64_t& lo, int64_t& hi) {
  const int64_t L = ((n + P - 1) / P + 31) & ~(int64_t)31;
  lo = (int64_t)c * L;
  hi = lo + L < n ? lo + L : n;
  if (lo > hi) lo = hi;
}

// Device-coherent word stores and loads (cache policy 16): histograms, bitmap words and cut
// keys handed to another workgroup of the same launch go through memory (written through,
// read around, the per-XCD L2s), ordered by waiting for the stores before the arrival
// counter moves.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t split_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__global__ __launch_bounds__(kThreadsK) void topk_split_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                                   const int32_t* __restrict__ lengths, int32_t k,
                                                                   int32_t P, SplitWs ws) {
  __shared__ SmemTopk sm;
  const int tid = threadIdx.x;
  const int32_t c = blockIdx.x;
  const int64_t t = blockIdx.y;
  const int64_t n = token_len(lengths, ld, t);
  if (n <= k) return;   // every workgroup of the token returns: the finish lists all positions
  int64_t lo, hi;
  split_chunk(n, P, c, lo, hi);
  const float* s = scores + t * ld + lo;
  radix_hist(sm, [&](auto f) { for_keys_global(s, hi - lo, f); }, 21, 2047u, 0u, 0u);
  const __amdgpu_buffer_rsrc_t rh = split_rsrc(ws.hist + (size_t)t * P * kBins, (uint32_t)P * kBins * 4);
  for (int i = tid; i < kBins; i += kThreadsK)
    __builtin_amdgcn_raw_buffer_store_b32(sm.hist[i], rh, (int)(4 * (c * kBins + i)), 0, 16);
  __builtin_amdgcn_s_waitcnt(0);   // the histogram is written through before the counter moves
  __syncthreads();
  if (tid == 0) {
    const int old = atomicAdd(&ws.arrive[t], 1);
    const uint32_t last = old == P - 1;
    if (last) atomicExch(&ws.arrive[t], 0);
    sm.pick[0] = last;
  }
  __syncthreads();
  const bool last = sm.pick[0] != 0;
  __syncthreads();
  if (!last) return;
  // the P histograms, eight chunks' loads in flight at a time for all of a thread's bins
  constexpr int kPer = kBins / kThreadsK;
  uint32_t sum[kPer] = {};
  for (int c0 = 0; c0 < P; c0 += 8) {
    uint32_t v[kPer][8];
#pragma unroll
    for (int j = 0; j < kPer; j++)
#pragma unroll
      for (int u = 0; u < 8; u++)
        v[j][u] = c0 + u < P ? __builtin_amdgcn_raw_buffer_load_b32(rh, (int)(4 * ((c0 + u) * kBins + tid + kThreadsK * j)), 0, 16)
                             : 0u;
#pragma unroll
    for (int j = 0; j < kPer; j++)
#pragma unroll
      for (int u = 0; u < 8; u++) sum[j] += v[j][u];
  }
#pragma unroll
  for (int j = 0; j < kPer; j++) sm.hist[tid + kThreadsK * j] = sum[j];
  __syncthreads();
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
  radix_pick(sm, 21, 2047u, prefix, pmask, need);
  if (tid == 0) {
    ws.rec[2 * t] = prefix >> 21;
    ws.rec[2 * t + 1] = need;
  }
}

__global__ __launch_bounds__(kThreadsK) void topk_split_classify_kernel(const float* __restrict__ scores, int64_t ld,
                                                                       const int32_t* __restrict__ lengths,
                                                                       const int32_t* __restrict__ row_offset,
                                                                       int32_t k, int32_t P, int32_t* __restrict__ out,
                                                                       SplitWs ws) {
  __shared__ SmemTopk sm;
  __shared__ uint32_t base;
  __shared__ int32_t bcast;
  const int tid = threadIdx.x;
  const int32_t c = blockIdx.x;
  const int64_t t = blockIdx.y;
  const int64_t n = token_len(lengths, ld, t);
  const int32_t off = row_offset ? row_offset[t] : 0;
  int32_t* o = out + t * (int64_t)k;
  if (n <= k) {   // every position, then empties: workgroup c writes entries c, c + P, ...
    for (int64_t p = (int64_t)c * kThreadsK + tid; p < k; p += (int64_t)P * kThreadsK) o[p] = p < n ? off + (int32_t)p : -1;
    return;
  }
  const int64_t W = (n + 31) >> 5;
  const bool in_lds = W <= kMapWords;   // else the finish reads the scores from memory
  const __amdgpu_buffer_rsrc_t rb = split_rsrc(ws.bmap + (size_t)t * kMapWords, kMapWords * 4);
  const __amdgpu_buffer_rsrc_t rk = split_rsrc(ws.ckey + (size_t)t * kCap, kCap * 4);
  const __amdgpu_buffer_rsrc_t rp = split_rsrc(ws.cpos + (size_t)t * kCap, kCap * 4);
  if (in_lds) {
    int64_t lo, hi;
    split_chunk(n, P, c, lo, hi);
    const int64_t m = hi - lo, nw = (m + 31) >> 5;
    for (int64_t i = tid; i < nw; i += kThreadsK) sm.above[i] = 0;
    __syncthreads();
    classify_pass(sm, scores + t * ld + lo, m, ws.rec[2 * t]);
    for (int64_t i = tid; i < nw; i += kThreadsK)
      __builtin_amdgcn_raw_buffer_store_b32(sm.above[i], rb, (int)(4 * ((lo >> 5) + i)), 0, 16);
    // the chunk's cut keys: a region that overflowed sends the token to the finish in memory
    uint32_t total = 0;
    bool over = false;
    for (int w = 0; w < kWavesK; w++) {
      over |= sm.wcut[w] > (uint32_t)kCapWave;
      total += sm.wcut[w];
    }
    if (tid == 0) base = (uint32_t)atomicAdd(&ws.ccount[t], over ? kCap + 1 : (int32_t)total);
    __syncthreads();
    if (!over && base + total <= (uint32_t)kCap) {
      for (int i = tid; i < kCap; i += kThreadsK) {
        const int w = i / kCapWave, r = i % kCapWave;
        if ((uint32_t)r >= sm.wcut[w]) continue;
        uint32_t before = 0;
        for (int v = 0; v < w; v++) before += sm.wcut[v];
        const int d = (int)(base + before + r);
        __builtin_amdgcn_raw_buffer_store_b32(sm.ckey[i], rk, 4 * d, 0, 16);
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(lo + sm.cpos[i]), rp, 4 * d, 0, 16);
      }
    }
  }
  // ---- the last of the token's workgroups finishes it
  __builtin_amdgcn_s_waitcnt(0);   // bitmap words and cut keys are written through first
  __syncthreads();
  if (tid == 0) {
    const int old = atomicAdd(&ws.arrive[t], 1);
    const int last = old == P - 1;
    if (last) {
      atomicExch(&ws.arrive[t], 0);
      bcast = atomicExch(&ws.ccount[t], 0);   // the cut keys of every chunk; zero for the next call
    } else {
      bcast = -1;
    }
  }
  __syncthreads();
  const int32_t cnt0 = bcast;
  if (cnt0 < 0) return;
  const int32_t cnt = in_lds ? cnt0 : kCap + 1;
  const uint32_t bin = ws.rec[2 * t], need = ws.rec[2 * t + 1];
  const uint32_t prefix = bin << 21, pmask = 2047u << 21;
  if (cnt <= kCap) {
    // every load of a thread issued before the first is used (bitmap words, keys, positions)
    constexpr int kBW = (kMapWords + kThreadsK - 1) / kThreadsK, kBC = kCap / kThreadsK;
    uint32_t wv[kBW], kv[kBC], pv[kBC];
#pragma unroll
    for (int j = 0; j < kBW; j++) {
      const int i = tid + kThreadsK * j;
      wv[j] = i < W ? __builtin_amdgcn_raw_buffer_load_b32(rb, 4 * i, 0, 16) : 0u;
    }
#pragma unroll
    for (int j = 0; j < kBC; j++) {
      const int i = tid + kThreadsK * j;
      kv[j] = i < cnt ? __builtin_amdgcn_raw_buffer_load_b32(rk, 4 * i, 0, 16) : 0u;
      pv[j] = i < cnt ? __builtin_amdgcn_raw_buffer_load_b32(rp, 4 * i, 0, 16) : 0u;
    }
#pragma unroll
    for (int j = 0; j < kBW; j++) {
      const int i = tid + kThreadsK * j;
      if (i < W) {
        sm.above[i] = wv[j];
        sm.tie[i] = 0;
      }
    }
#pragma unroll
    for (int j = 0; j < kBC; j++) {
      const int i = tid + kThreadsK * j;
      if (i < cnt) {
        sm.ckey[i] = kv[j];
        sm.cpos[i] = (int32_t)pv[j];
      }
    }
    __syncthreads();
    finish_in_lds(sm, [&](int i) { return i < cnt; }, prefix, pmask, need, W, off, o, k);
  } else {
    finish_in_memory(sm, scores + t * ld, n, prefix, pmask, need, off, o, k);
  }
}

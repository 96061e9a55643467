// Body of the top-k selection (see indexer.hip), included once per workgroup size: the
// including file defines kThreadsK (threads per workgroup) in the enclosing namespace.
// No include guard: each inclusion instantiates the code in its own namespace.

constexpr int kWavesK = kThreadsK / 64;
constexpr int kBins = 2048;
constexpr int kMaxK = 65536;
constexpr int kVec = 4;                         // 16-byte loads per thread per round
constexpr int kRound = 4 * kVec * kThreadsK;    // positions per round
constexpr int kCap = 4096;                      // keys of the cut bin kept in LDS
constexpr int kCapWave = kCap / (kThreadsK / 64);   // each wave fills a region of its own
constexpr int kMapWords = 4608;                 // position bitmap words: contexts up to 147,456
static_assert(kBins % kThreadsK == 0, "every thread holds the same number of bins");

struct SmemTopk {
  uint32_t hist[kBins];
  uint32_t above[kMapWords];   // bit p: position p is in the list for certain (key above K)
  uint32_t tie[kMapWords];     // bit p: key of position p equals K
  uint32_t ckey[kCap];         // keys of the cut bin: wave w's in [w kCapWave, (w + 1) kCapWave)
  int32_t cpos[kCap];          // their positions
  uint32_t wsum[kWavesK];
  uint32_t wcut[kWavesK];      // keys of the cut bin each wave found
  uint32_t pick[2];            // chosen bin, keys above it
};

// Unsigned order of the key = numeric order of the score; -0 maps to the key of +0 (adding
// +0 turns -0 into +0 and leaves every other value, subnormals included, as it is).  No
// compares: a negative score's bits are inverted, a positive one's sign bit is set.
__device__ __forceinline__ uint32_t score_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
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

// Keys of positions p .. p + 3 (those below n) into key[0..3]; absent ones are not used.
__device__ __forceinline__ void load4(const float* __restrict__ s, int64_t p, int64_t n, uint32_t* key) {
  if (p + 3 < n) {
    const float4 v = *(const float4*)(s + p);
    key[0] = score_key(v.x);
    key[1] = score_key(v.y);
    key[2] = score_key(v.z);
    key[3] = score_key(v.w);
  } else {
#pragma unroll
    for (int j = 0; j < 4; j++) key[j] = p + j < n ? score_key(s[p + j]) : 0u;
  }
}

// Keys of the 4 kVec positions a thread takes in a round: 16-byte loads at p + 4 j * stride
// (j < kVec), all issued before any is used.  A full round (every position below n) loads
// without tests, so nothing stands between the loads; the last round tests each position.
template <bool kFull>
__device__ __forceinline__ void load_round(const float* __restrict__ s, int64_t p, int64_t stride, int64_t n,
                                           uint32_t (&key)[4 * kVec]) {
  if constexpr (kFull) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    f4 v[kVec];
#pragma unroll
    for (int j = 0; j < kVec; j++) v[j] = *(const f4*)(s + p + 4 * j * stride);
    __builtin_amdgcn_sched_barrier(0);   // every load is issued before any is used
#pragma unroll
    for (int j = 0; j < kVec; j++) {
      key[4 * j + 0] = score_key(v[j].x);
      key[4 * j + 1] = score_key(v[j].y);
      key[4 * j + 2] = score_key(v[j].z);
      key[4 * j + 3] = score_key(v[j].w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kVec; j++) load4(s, p + 4 * j * stride, n, key + 4 * j);
  }
}

// Raw 16-byte loads of a full round (positions p + 4 j stride, j < kVec), issued together.
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void issue_round(const float* __restrict__ s, int64_t p, int64_t stride,
                                            f4v (&v)[kVec]) {
#pragma unroll
  for (int j = 0; j < kVec; j++) v[j] = *(const f4v*)(s + p + 4 * j * stride);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void keys_of(const f4v (&v)[kVec], uint32_t (&key)[4 * kVec]) {
#pragma unroll
  for (int j = 0; j < kVec; j++) {
    key[4 * j + 0] = score_key(v[j].x);
    key[4 * j + 1] = score_key(v[j].y);
    key[4 * j + 2] = score_key(v[j].z);
    key[4 * j + 3] = score_key(v[j].w);
  }
}

// g(key[], c, full) for every round of the token: thread tid takes the 16-byte pieces tid,
// tid + kThreadsK, ... of each round (every load instruction of a wave reads 1 KB of
// consecutive scores).  Two register buffers: the loads of round r + 1 are in flight while
// round r is processed.  The last, partial round tests each position.
template <class G>
__device__ __forceinline__ void for_rounds(const float* __restrict__ s, int64_t n, G g) {
  const int tid = threadIdx.x;
  const int64_t rounds = n / kRound;
  const int64_t p = 4 * tid;
  f4v a[kVec], b[kVec];
  uint32_t key[4 * kVec];
  if (rounds > 0) issue_round(s, p, kThreadsK, a);
  for (int64_t r = 0; r < rounds; r += 2) {
    if (r + 1 < rounds) issue_round(s, (r + 1) * kRound + p, kThreadsK, b);
    keys_of(a, key);
    g(key, r * kRound, true);
    if (r + 1 >= rounds) break;
    if (r + 2 < rounds) issue_round(s, (r + 2) * kRound + p, kThreadsK, a);
    keys_of(b, key);
    g(key, (r + 1) * kRound, true);
  }
  const int64_t c = rounds * kRound;
  if (c < n) {
    load_round<false>(s, c + p, kThreadsK, n, key);
    g(key, c, false);
  }
}

// f(key, position) for every key of the token (not in position order).
template <class F>
__device__ __forceinline__ void for_keys_global(const float* __restrict__ s, int64_t n, F f) {
  const int tid = threadIdx.x;
  for_rounds(s, n, [&](const uint32_t (&key)[4 * kVec], int64_t c, bool full) {
#pragma unroll
    for (int j = 0; j < kVec; j++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int64_t q = c + 4 * (tid + (int64_t)kThreadsK * j) + e;
        if (full || q < n) f(key[4 * j + e], q);
      }
  });
}

// Histogram, in sm.hist, of bits shift .. shift + log2(bmask + 1) of the keys that match
// `prefix` under `pmask`; `visit(f)` calls f(key, position) for every key.
template <class V>
__device__ __forceinline__ void radix_hist(SmemTopk& sm, V visit, int shift, uint32_t bmask, uint32_t prefix,
                                           uint32_t pmask) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kBins; i += kThreadsK) sm.hist[i] = 0;
  __syncthreads();
  const uint32_t pf = prefix, pm = pmask;
  visit([&](uint32_t key, int64_t) {
    if ((key & pm) == pf) atomicAdd(&sm.hist[(key >> shift) & bmask], 1u);
  });
  __syncthreads();
}

// The bin of sm.hist (bins 0 .. bmask) holding the need-th largest key; narrows prefix /
// pmask and takes the keys of higher bins off `need`.
__device__ __forceinline__ void radix_pick(SmemTopk& sm, int shift, uint32_t bmask, uint32_t& prefix,
                                           uint32_t& pmask, uint32_t& need) {
  const int tid = threadIdx.x;
  // thread tid holds the kPerBins bins of descending rank kPerBins tid .. + kPerBins - 1
  constexpr int kPerBins = kBins / kThreadsK;
  uint32_t h[kPerBins], sum = 0;
#pragma unroll
  for (int i = 0; i < kPerBins; i++) {
    const int b = (int)bmask - kPerBins * tid - i;
    h[i] = b >= 0 ? sm.hist[b] : 0u;
    sum += h[i];
  }
  uint32_t tot;
  uint32_t before = block_scan(sm, sum, tot) - sum;   // keys in higher bins
#pragma unroll
  for (int i = 0; i < kPerBins; i++) {
    if (before < need && need <= before + h[i]) {   // true for exactly one bin of the workgroup
      sm.pick[0] = (uint32_t)((int)bmask - kPerBins * tid - i);
      sm.pick[1] = before;
    }
    before += h[i];
  }
  __syncthreads();
  prefix |= sm.pick[0] << shift;
  pmask |= bmask << shift;
  need -= sm.pick[1];
  __syncthreads();
}

// One radix step: the histogram, then the bin of the need-th largest key.
template <class V>
__device__ __forceinline__ void radix_step(SmemTopk& sm, V visit, int shift, uint32_t bmask, uint32_t& prefix,
                                           uint32_t& pmask, uint32_t& need) {
  radix_hist(sm, visit, shift, bmask, prefix, pmask);
  radix_pick(sm, shift, bmask, prefix, pmask, need);
}

// The list from `cnt` (key, position) pairs in position order, given by at(i, key, pos):
// every key above K and the first `need` keys equal to K.  gb / eb count the keys above K /
// equal to K before a pair; its place is gb + min(eb, need).  The places are below k by
// construction; the test only keeps a write inside the token's row.
template <class A>
__device__ __forceinline__ void emit(SmemTopk& sm, int64_t cnt, A at, uint32_t K, uint32_t need, int32_t off,
                                     int32_t* __restrict__ o, int32_t k) {
  const int tid = threadIdx.x;
  uint32_t gt_run = 0, eq_run = 0;
  for (int64_t c = 0; c < cnt; c += 4 * kThreadsK) {
    const int64_t i0 = c + 4 * tid;
    uint32_t key[4];
    int32_t pos[4];
    at(i0, key, pos);
    uint32_t g = 0, e = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      g += (i0 + j < cnt && key[j] > K) ? 1u : 0u;
      e += (i0 + j < cnt && key[j] == K) ? 1u : 0u;
    }
    const uint32_t mine = g | (e << 16);   // at most 4 kThreadsK of each per chunk
    uint32_t tot;
    const uint32_t excl = block_scan(sm, mine, tot) - mine;
    uint32_t gb = gt_run + (excl & 0xFFFFu), eb = eq_run + (excl >> 16);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (i0 + j >= cnt) continue;
      const int32_t entry = off + pos[j];
      if (key[j] > K) {
        const uint32_t place = gb + (eb < need ? eb : need);
        if (place < (uint32_t)k) o[place] = entry;
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

// Pass 2 over the n scores at s (positions relative to s): keys in bins above `cut` set
// their bits in sm.above (word p >> 5); keys in bin `cut` go with their positions to their
// wave's region of sm.ckey / sm.cpos.  Afterwards sm.wcut[w] holds the keys of the cut bin
// wave w found (more than kCapWave: its region overflowed).  sm.above must be zero.
__device__ __forceinline__ void classify_pass(SmemTopk& sm, const float* __restrict__ s, int64_t n, uint32_t cut) {
  const int tid = threadIdx.x;
  // opaque to the optimizer, which would otherwise turn the sign-bit tests below back into
  // compare-and-select pairs
  asm volatile("" : "+v"(cut));
  const int wave = tid >> 6;
  uint32_t wfill = 0;   // keys of the cut bin this wave found so far (uniform in the wave)
  // one round.  The 4 positions of a 16-byte load share one bitmap word (they start at a
  // multiple of 4), so each load sets its bits with one OR (of 0 when none is above the
  // cut).  A lane's cut-bin keys go to its wave's region after those of lower lanes: the
  // wave prefix sum of the counts (below 32) is built from ballots of their five bits.
  auto round = [&](const uint32_t (&key)[4 * kVec], int64_t c, bool full) {
    uint32_t cutm[kVec], m = 0;
#pragma unroll
    for (int j = 0; j < kVec; j++) {
      const int64_t p = c + 4 * (tid + (int64_t)kThreadsK * j);
      uint32_t am = 0, cm = 0;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        // bins are below 2^11: cut - b is negative exactly when b > cut, and
        // (b ^ cut) - 1 exactly when b == cut
        const uint32_t b = key[4 * j + e] >> 21;
        uint32_t above = (cut - b) >> 31, equal = ((b ^ cut) - 1u) >> 31;
        if (!full && p + e >= n) above = equal = 0;
        am |= above << e;
        cm |= equal << e;
      }
      if (p < n) atomicOr(&sm.above[p >> 5], am << (p & 31));
      cutm[j] = cm;
      m += __builtin_popcount(cm);
    }
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int bit = 0; bit < 5; bit++) {
      const uint64_t bal = __ballot((m >> bit) & 1u);
      before += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))
                << bit;
      total += (uint32_t)__popcll(bal) << bit;
    }
    if (m != 0) {
      uint32_t i = wfill + before;
#pragma unroll
      for (int j = 0; j < kVec; j++) {
        if (cutm[j] == 0) continue;
        const int64_t p = c + 4 * (tid + (int64_t)kThreadsK * j);
#pragma unroll
        for (int e = 0; e < 4; e++) {
          if ((cutm[j] >> e) & 1u) {
            if (i < (uint32_t)kCapWave) {
              sm.ckey[wave * kCapWave + i] = key[4 * j + e];
              sm.cpos[wave * kCapWave + i] = (int32_t)(p + e);
            }
            i++;
          }
        }
      }
    }
    wfill += total;
  };
  for_rounds(s, n, round);
  if ((tid & 63) == 0) sm.wcut[wave] = wfill;
  __syncthreads();
}

// The rest of the selection in LDS, once pass 1 has picked the top-11-bit bin (prefix /
// pmask / need): the keys above that bin are bits of sm.above[0, W), the cut bin's keys and
// positions are in sm.ckey / sm.cpos (entry i holds one when kept(i)), sm.tie is zero.  The
// two remaining radix steps give K and how many keys equal to K the list takes; the list is
// written in position order from the bitmaps.
template <class Kept>
__device__ __forceinline__ void finish_in_lds(SmemTopk& sm, Kept kept, uint32_t prefix, uint32_t pmask, uint32_t need,
                                              int64_t W, int32_t off, int32_t* __restrict__ o, int32_t k) {
  const int tid = threadIdx.x;
  auto lds_keys = [&](auto f) {
    for (int i = tid; i < kCap; i += kThreadsK)
      if (kept(i)) f(sm.ckey[i], (int64_t)0);
  };
  radix_step(sm, lds_keys, 10, 2047u, prefix, pmask, need);
  radix_step(sm, lds_keys, 0, 1023u, prefix, pmask, need);
  const uint32_t K = prefix;
  for (int i = tid; i < kCap; i += kThreadsK) {
    if (!kept(i)) continue;
    const uint32_t key = sm.ckey[i];
    const int32_t p = sm.cpos[i];
    if (key > K) atomicOr(&sm.above[p >> 5], 1u << (p & 31));
    else if (key == K) atomicOr(&sm.tie[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  // ---- the list from the bitmaps: thread tid takes words [w0, w1); a set bit of `above`
  // goes to gb + min(eb, need), one of `tie` to gb + eb while eb < need (gb / eb: bits of
  // `above` / `tie` at lower positions)
  const int per = (int)((W + kThreadsK - 1) / kThreadsK);
  const int w0 = tid * per, w1 = (int)(w0 + per < W ? w0 + per : W);
  uint32_t g = 0, e = 0;
  for (int w = w0; w < w1; w++) {
    g += __builtin_popcount(sm.above[w]);
    e += __builtin_popcount(sm.tie[w]);
  }
  uint32_t tot;
  uint32_t gb = block_scan(sm, g, tot) - g;
  uint32_t eb = block_scan(sm, e, tot) - e;
  for (int w = w0; w < w1; w++) {
    const uint32_t a = sm.above[w], t = sm.tie[w];
    uint32_t m = a | t;
    while (m) {
      const int bit = __builtin_ctz(m);
      m &= m - 1;
      const int32_t entry = off + (w * 32 + bit);
      // the places are below k by construction; the test only keeps a write inside the row
      if ((a >> bit) & 1u) {
        const uint32_t place = gb + (eb < need ? eb : need);
        if (place < (uint32_t)k) o[place] = entry;
        gb++;
      } else {
        if (eb < need && gb + eb < (uint32_t)k) o[gb + eb] = entry;
        eb++;
      }
    }
  }
}

// The same from the n scores at s in memory: a context longer than the bitmaps, or a cut bin
// with more keys than LDS keeps.
__device__ __forceinline__ void finish_in_memory(SmemTopk& sm, const float* __restrict__ s, int64_t n,
                                                 uint32_t prefix, uint32_t pmask, uint32_t need, int32_t off,
                                                 int32_t* __restrict__ o, int32_t k) {
  auto global_keys = [&](auto f) { for_keys_global(s, n, f); };
  radix_step(sm, global_keys, 10, 2047u, prefix, pmask, need);
  radix_step(sm, global_keys, 0, 1023u, prefix, pmask, need);
  emit(sm, n,
       [&](int64_t i0, uint32_t* key, int32_t* pos) {
         load4(s, i0, n, key);
#pragma unroll
         for (int j = 0; j < 4; j++) pos[j] = (int32_t)(i0 + j);
       },
       prefix, need, off, o, k);
}

// Positions of token t (lengths clamped to [0, ld]).
__device__ __forceinline__ int64_t token_len(const int32_t* __restrict__ lengths, int64_t ld, int64_t t) {
  const int64_t n = lengths ? (int64_t)lengths[t] : ld;
  return n < 0 ? 0 : (n > ld ? ld : n);
}

__global__ __launch_bounds__(kThreadsK) void sparse_indexer_topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                                       const int32_t* __restrict__ lengths,
                                                                       const int32_t* __restrict__ row_offset,
                                                                       int32_t k, int32_t* __restrict__ out) {
  __shared__ SmemTopk sm;
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int64_t n = token_len(lengths, ld, t);
  const int32_t off = row_offset ? row_offset[t] : 0;
  const float* s = scores + t * ld;
  int32_t* o = out + t * (int64_t)k;
  if (n <= k) {   // every position, then empties
    for (int p = tid; p < k; p += kThreadsK) o[p] = p < n ? off + p : -1;
    return;
  }
  auto global_keys = [&](auto f) { for_keys_global(s, n, f); };

  // ---- pass 1: the top-11-bit bin of the k-th key
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
  radix_step(sm, global_keys, 21, 2047u, prefix, pmask, need);

  const int64_t W = (n + 31) >> 5;   // bitmap words of the context
  uint32_t cnt = kCap + 1;
  if (W <= kMapWords) {
    // ---- pass 2: keys above the cut bin are in the list: set their bits; keys in the cut
    // bin go to LDS with their positions
    for (int64_t i = tid; i < W; i += kThreadsK) {
      sm.above[i] = 0;
      sm.tie[i] = 0;
    }
    __syncthreads();
    classify_pass(sm, s, n, prefix >> 21);
    cnt = 0;
    for (int w = 0; w < kWavesK; w++) cnt = sm.wcut[w] > (uint32_t)kCapWave ? (uint32_t)kCap + 1 : cnt + sm.wcut[w];
  }
  if (cnt <= (uint32_t)kCap) {
    // entry i of the buffer holds a key when it lies below its wave's fill
    finish_in_lds(sm, [&](int i) { return (uint32_t)(i % kCapWave) < sm.wcut[i / kCapWave]; }, prefix, pmask,
                  need, W, off, o, k);
  } else {
    finish_in_memory(sm, s, n, prefix, pmask, need, off, o, k);
  }
}

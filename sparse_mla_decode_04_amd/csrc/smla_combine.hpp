// Log-sum-exp merge of split results for one token and a block of NH heads (16 or 32),
// run by a team of 256 threads (a whole workgroup, or one half of a 512-thread one; `tid`
// is the thread's index in the team).  Used by the standalone combine kernel and by the last
// workgroup of a token inside the decode kernel.
//
// Each split s holds its normalized output O_s[NH][512] (fp32, head stride 512 floats) and
// its natural-log LSE lse_s[NH].  lse = ln sum_s exp(lse_s); out = sum_s exp(lse_s - lse) O_s.
// A split with lse_s = -inf has weight zero; if every split is -inf the output is zero and
// lse = -inf.  (The split of the work follows from sizing the decomposition by the token
// batch: "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section
// "Four-bit caches make room".)
//
// The partials are read through a buffer resource: with kCoherent the loads use the
// device-coherent policy (partials written by other workgroups of the same launch, through
// other XCDs' L2), otherwise the default one.  The loads of several splits are issued
// together, so the merge costs a few memory latencies rather than one per split.
#pragma once

#include "smla_device.hpp"

namespace smla {

// Buffer resource over [base, base + bytes), raw byte addressing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t merge_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

template <bool kCoherent>
__device__ __forceinline__ float merge_ld1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kCoherent ? 16 : 0));
}
template <bool kCoherent>
__device__ __forceinline__ f32x4 merge_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoherent ? 16 : 0));
}

// The eight XCDs of MI355X each have a private L2.  Partial results that one workgroup hands
// to another inside a launch are written with the device-coherent policy (sc1: written
// through the private L2 to memory) and read with it (read around the private L2); the
// hand-off is ordered by waiting for the stores to complete before the counter update, so
// no L2 write-back or invalidate is needed.  One 16-byte store per piece: split into smaller
// stores, each piece would cost several partial-line writes.
__device__ __forceinline__ void merge_st4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 16);
}
__device__ __forceinline__ void merge_st1(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 16);
}

// active = false: the thread does no work but passes the same barriers (a team that
// shares the workgroup with the merging one).
//
// part(s, &o_off, &l_off): byte offsets of split s's O[NH][512] within the buffer of `ro`
// and of its lse[NH] within the buffer of `rl`.  out: head 0 of the block (head stride 512
// fp16); lse_out: head 0.  scratch: >= 2048 floats of LDS.
//
// More splits than 256 / NH: phase 1, per-head running maximum and denominator of the LSEs,
// folded by all threads and reduced through LDS.  Phase 2, per chunk of up to 32 splits: the weights
// exp(lse_s - lse) go to LDS, then the outputs are summed with every load instruction of a
// wave reading 1 KB of consecutive bytes (thread tid takes 16-byte pieces tid, tid+256, ...
// of the NH x 512 block, so one thread covers several heads).
//
// Few splits (ns <= SMAX): every thread loads the LSEs of its own heads and its output
// pieces of every split at once -- one memory round trip -- and computes the weights of
// its heads itself.
template <int NH, int SMAX, bool kCoherent, class PartFn>
__device__ __forceinline__ void lse_merge_few(int ns, __amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rl,
                                              PartFn part, f16* out, float* lse_out, int tid) {
  constexpr int P = NH / 2;   // 16-byte pieces per thread: piece q is head (256q + tid) / 128
  const int h1 = tid >> 7;    // head of piece q is 2q + h1
  float ls[SMAX][P];
  f32x4 ov[SMAX][P];
#pragma unroll
  for (int s = 0; s < SMAX; s++) {
    uint32_t o_off, l_off;
    part(s < ns ? s : 0, &o_off, &l_off);
#pragma unroll
    for (int q = 0; q < P; q++) {
      ls[s][q] = merge_ld1<kCoherent>(rl, l_off + 4u * (2 * q + h1));
      ov[s][q] = merge_ld4<kCoherent>(ro, o_off + 16u * (256 * q + tid));
    }
  }
#pragma unroll
  for (int q = 0; q < P; q++) {
    float m = -INFINITY;
#pragma unroll
    for (int s = 0; s < SMAX; s++)
      if (s < ns) m = fmaxf(m, ls[s][q]);
    float d = 0.0f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (m != -INFINITY) {
#pragma unroll
      for (int s = 0; s < SMAX; s++) {
        if (s < ns && ls[s][q] != -INFINITY) {
          const float wgt = __expf(ls[s][q] - m);
          d += wgt;
          acc += wgt * ov[s][q];
        }
      }
    }
    const float inv = d > 0.0f ? 1.0f / d : 0.0f;
    const int e = 256 * q + tid, h = e / 128, col = 4 * (e % 128);
    const f32x4 v = acc * inv;
    *(f16x4*)(out + 512 * h + col) = f16x4{(f16)v.x, (f16)v.y, (f16)v.z, (f16)v.w};
    if ((e % 128) == 0) lse_out[h] = d > 0.0f ? m + logf(d) : -INFINITY;
  }
}

// 32 heads, up to 2U = 4 splits: the LSEs of every split (one value per
// thread) and the output pieces of the first U splits in one memory round trip; the
// per-head maximum, denominator and split weights through LDS; the output pieces of the
// other splits in a second round trip.
template <int NH, int U, bool kCoherent, class PartFn>
__device__ __forceinline__ void lse_merge_two(int ns, __amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rl,
                                              PartFn part, f16* out, float* lse_out, float* scratch, int tid,
                                              bool active) {
  constexpr int P = NH / 2;             // 16-byte pieces per thread: piece q is head 2q + tid / 128
  static_assert(2 * U * NH <= 256, "one LSE per thread");
  float* const ls = scratch;            // [2U][NH] LSEs (-inf beyond ns)
  float* const wt = scratch + 256;      // [2U][NH] weights
  float* const mh = scratch + 512;      // [NH] maximum
  float* const ih = scratch + 512 + NH; // [NH] 1 / denominator
  const int h1 = tid >> 7;
  f32x4 ov[U][P];
  if (active) {
    float x = -INFINITY;
    if (tid < ns * NH) {
      uint32_t o_off, l_off;
      part(tid / NH, &o_off, &l_off);
      x = merge_ld1<kCoherent>(rl, l_off + 4u * (tid % NH));
    }
#pragma unroll
    for (int u = 0; u < U; u++) {   // ns > U: every one of these splits exists
      uint32_t o_off, l_off;
      part(u, &o_off, &l_off);
#pragma unroll
      for (int q = 0; q < P; q++) ov[u][q] = merge_ld4<kCoherent>(ro, o_off + 16u * (256 * q + tid));
    }
    if (tid < 2 * U * NH) ls[tid] = x;
  }
  __syncthreads();
  if (active && tid < NH) {
    float m = -INFINITY;
#pragma unroll
    for (int s = 0; s < 2 * U; s++) m = fmaxf(m, ls[s * NH + tid]);
    float d = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
      for (int s = 0; s < 2 * U; s++) {
        const float l = ls[s * NH + tid];
        if (l != -INFINITY) d += __expf(l - m);
      }
    }
    mh[tid] = m;
    ih[tid] = d > 0.0f ? 1.0f / d : 0.0f;
    lse_out[tid] = d > 0.0f ? m + logf(d) : -INFINITY;
  }
  __syncthreads();
  if (active && tid < 2 * U * NH) {
    const int h = tid % NH;
    const float l = ls[tid];
    wt[tid] = (l == -INFINITY) ? 0.0f : __expf(l - mh[h]) * ih[h];
  }
  __syncthreads();
  if (!active) return;
  f32x4 acc[P];
#pragma unroll
  for (int q = 0; q < P; q++) {
    acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < U; u++) acc[q] += wt[u * NH + 2 * q + h1] * ov[u][q];
  }
#pragma unroll
  for (int u = 0; u < U; u++) {
    const int s = U + u;
    uint32_t o_off, l_off;
    part(s < ns ? s : 0, &o_off, &l_off);
#pragma unroll
    for (int q = 0; q < P; q++) ov[u][q] = merge_ld4<kCoherent>(ro, o_off + 16u * (256 * q + tid));
  }
#pragma unroll
  for (int u = 0; u < U; u++) {
    if (U + u >= ns) continue;
#pragma unroll
    for (int q = 0; q < P; q++) acc[q] += wt[(U + u) * NH + 2 * q + h1] * ov[u][q];
  }
#pragma unroll
  for (int q = 0; q < P; q++) {
    const int e = 256 * q + tid, h = e / 128, col = 4 * (e % 128);
    *(f16x4*)(out + 512 * h + col) = f16x4{(f16)acc[q].x, (f16)acc[q].y, (f16)acc[q].z, (f16)acc[q].w};
  }
}

// 16 heads, up to 16 splits: the LSEs of every split (one value per thread) and the output
// pieces of the first U splits in one memory round trip; the per-head maximum, denominator
// and split weights through LDS; the output pieces of the other splits in batches of U, one
// round trip each.
template <int NH, int U, bool kCoherent, class PartFn>
__device__ __forceinline__ void lse_merge_batched(int ns, __amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rl,
                                                  PartFn part, f16* out, float* lse_out, float* scratch, int tid,
                                                  bool active) {
  constexpr int P = NH / 2;             // 16-byte pieces per thread: piece q is head 2q + tid / 128
  constexpr int SMAX = 256 / NH;        // splits whose LSEs one value per thread covers
  float* const ls = scratch;            // [SMAX][NH] LSEs (-inf beyond ns)
  float* const wt = scratch + 256;      // [SMAX][NH] weights
  float* const mh = scratch + 512;      // [NH] maximum
  float* const ih = scratch + 512 + NH; // [NH] 1 / denominator
  const int h1 = tid >> 7;
  f32x4 ov[U][P];
  if (active) {
    float x = -INFINITY;
    if (tid < ns * NH) {
      uint32_t o_off, l_off;
      part(tid / NH, &o_off, &l_off);
      x = merge_ld1<kCoherent>(rl, l_off + 4u * (tid % NH));
    }
#pragma unroll
    for (int u = 0; u < U; u++) {   // ns > U: every one of these splits exists
      uint32_t o_off, l_off;
      part(u, &o_off, &l_off);
#pragma unroll
      for (int q = 0; q < P; q++) ov[u][q] = merge_ld4<kCoherent>(ro, o_off + 16u * (256 * q + tid));
    }
    ls[tid] = x;
  }
  __syncthreads();
  if (active && tid < NH) {
    float m = -INFINITY;
#pragma unroll
    for (int s = 0; s < SMAX; s++) m = fmaxf(m, ls[s * NH + tid]);
    float d = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
      for (int s = 0; s < SMAX; s++) {
        const float l = ls[s * NH + tid];
        if (l != -INFINITY) d += __expf(l - m);
      }
    }
    mh[tid] = m;
    ih[tid] = d > 0.0f ? 1.0f / d : 0.0f;
    lse_out[tid] = d > 0.0f ? m + logf(d) : -INFINITY;
  }
  __syncthreads();
  if (active) {
    const int h = tid % NH;
    const float l = ls[tid];
    wt[tid] = (l == -INFINITY) ? 0.0f : __expf(l - mh[h]) * ih[h];
  }
  __syncthreads();
  if (!active) return;
  f32x4 acc[P];
#pragma unroll
  for (int q = 0; q < P; q++) {
    acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < U; u++) acc[q] += wt[u * NH + 2 * q + h1] * ov[u][q];
  }
  static_assert(NH == 16, "16 heads");
  constexpr int kMaxBatches = SMAX / U - 1;   // batches after the first
#pragma unroll
  for (int bi = 0; bi < kMaxBatches; bi++) {
    const int b = U * (bi + 1);
    if (b >= ns) break;
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int s = b + u;
      uint32_t o_off, l_off;
      part(s < ns ? s : 0, &o_off, &l_off);
#pragma unroll
      for (int q = 0; q < P; q++) ov[u][q] = merge_ld4<kCoherent>(ro, o_off + 16u * (256 * q + tid));
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (b + u >= ns) continue;
#pragma unroll
      for (int q = 0; q < P; q++) acc[q] += wt[(b + u) * NH + 2 * q + h1] * ov[u][q];
    }
  }
#pragma unroll
  for (int q = 0; q < P; q++) {
    const int e = 256 * q + tid, h = e / 128, col = 4 * (e % 128);
    *(f16x4*)(out + 512 * h + col) = f16x4{(f16)acc[q].x, (f16)acc[q].y, (f16)acc[q].z, (f16)acc[q].w};
  }
}

template <int NH, bool kCoherent, class PartFn>
__device__ __forceinline__ void lse_merge(int ns, __amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rl,
                                          PartFn part, f16* out, float* lse_out, float* scratch, int tid,
                                          bool active = true) {
  static_assert(NH == 16 || NH == 32, "head block");
  constexpr int kFew = NH == 16 ? 4 : 2;
  constexpr int U = NH == 16 ? 4 : 2;  // splits per batch of output loads
  if (ns <= kFew) {
    if (active) lse_merge_few<NH, kFew, kCoherent>(ns, ro, rl, part, out, lse_out, tid);
    return;
  }
  if constexpr (NH == 16) {
    if (ns <= 256 / NH) {
      lse_merge_batched<NH, U, kCoherent>(ns, ro, rl, part, out, lse_out, scratch, tid, active);
      return;
    }
  } else {
    if (ns <= 2 * U) {
      lse_merge_two<NH, U, kCoherent>(ns, ro, rl, part, out, lse_out, scratch, tid, active);
      return;
    }
  }
  constexpr int K = 256 / NH;          // threads per head in phase 1
  constexpr int P = NH / 2;            // 16-byte pieces per thread per split (NH*512*4 / 4096)
  constexpr int CS = 32;               // splits per chunk of weights
  float* const red = scratch;                 // [2][256] phase-1 partials
  float* const mh = scratch + 512;            // [NH] maximum
  float* const ih = scratch + 512 + NH;       // [NH] 1 / denominator
  float* const wt = scratch + 1024;           // [CS][NH] weights of a chunk

  // ---- phase 1: thread (h, k) folds splits k, k+K, ...
  if (active) {
    const int h = tid % NH, k = tid / NH;
    float m = -INFINITY, d = 0.0f;
    for (int s0 = 0; s0 < ns; s0 += 4 * K) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int s = s0 + u * K + k;
        uint32_t o_off, l_off;
        part(s < ns ? s : 0, &o_off, &l_off);
        const float x = merge_ld1<kCoherent>(rl, l_off + 4u * h);
        v[u] = s < ns ? x : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        if (v[u] == -INFINITY) continue;
        if (v[u] > m) {
          d = d * __expf(m - v[u]) + 1.0f;   // exp(-inf) = 0 on the first value
          m = v[u];
        } else {
          d += __expf(v[u] - m);
        }
      }
    }
    red[tid] = m;
    red[256 + tid] = d;
  }
  __syncthreads();
  if (active && tid < NH) {
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < K; k++) m = fmaxf(m, red[k * NH + tid]);
    float d = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
      for (int k = 0; k < K; k++) {
        const float mk = red[k * NH + tid];
        if (mk != -INFINITY) d += red[256 + k * NH + tid] * __expf(mk - m);
      }
    }
    mh[tid] = m;
    ih[tid] = d > 0.0f ? 1.0f / d : 0.0f;
    lse_out[tid] = d > 0.0f ? m + logf(d) : -INFINITY;
  }
  __syncthreads();

  // ---- phase 2: piece q of thread tid holds floats 4*(256q + tid) .. +3 of the block,
  // i.e. head (256q + tid) / 128, columns 4 * ((256q + tid) % 128) ..
  f32x4 acc[P];
#pragma unroll
  for (int q = 0; q < P; q++) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < ns; c0 += CS) {
    const int cn = min(CS, ns - c0);
    for (int e = tid; active && e < cn * NH; e += 256) {
      const int s = e / NH, h = e - s * NH;
      uint32_t o_off, l_off;
      part(c0 + s, &o_off, &l_off);
      const float ls = merge_ld1<kCoherent>(rl, l_off + 4u * h);
      wt[e] = (ls == -INFINITY) ? 0.0f : __expf(ls - mh[h]) * ih[h];
    }
    __syncthreads();
    for (int s0 = 0; active && s0 < cn; s0 += U) {
      f32x4 ov[U][P];
#pragma unroll
      for (int u = 0; u < U; u++) {
        uint32_t o_off, l_off;
        part(c0 + (s0 + u < cn ? s0 + u : 0), &o_off, &l_off);
#pragma unroll
        for (int q = 0; q < P; q++) ov[u][q] = merge_ld4<kCoherent>(ro, o_off + 16u * (256 * q + tid));
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        if (s0 + u >= cn) continue;
#pragma unroll
        for (int q = 0; q < P; q++) acc[q] += wt[(s0 + u) * NH + (256 * q + tid) / 128] * ov[u][q];
      }
    }
    __syncthreads();
  }
  if (!active) return;
#pragma unroll
  for (int q = 0; q < P; q++) {
    const int e = 256 * q + tid, h = e / 128, col = 4 * (e % 128);
    *(f16x4*)(out + 512 * h + col) = f16x4{(f16)acc[q].x, (f16)acc[q].y, (f16)acc[q].z, (f16)acc[q].w};
  }
}

}  // namespace smla

// Log-sum-exp merge of split results for one token and one group of 16 heads, run by a
// 256-thread workgroup.  Used by the standalone combine kernel and by the last
// workgroup of a token inside the decode kernel.
//
// Each split s holds its normalized output O_s[16][512] (fp32, head stride 512) and its
// natural-log LSE lse_s[16].  lse = ln sum_s exp(lse_s); out = sum_s exp(lse_s - lse) O_s.
// A split with lse_s = -inf has weight zero; if every split is -inf the output is zero and
// lse = -inf.  (The split of the work follows from sizing the decomposition by the token
// batch: "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section
// "Four-bit caches make room".)
#pragma once

#include "smla_device.hpp"

namespace smla {

// part(s, &o, &l) yields the fp32 [16][512] output and the [16] LSE of split s.
// out points at head 0 of the group (head stride out_hstride fp16 elements); lse at head 0.
// kCoherent: the partials were written by other workgroups of the same launch (read them
// with device-coherent loads); false when they come from an earlier launch.
// Thread tid owns head tid/16 and columns 32*(tid%16) .. +31.  The loads of a batch of
// splits are issued together so that the merge costs a few memory latencies, not one per
// split.
template <bool kCoherent, class PartFn>
__device__ __forceinline__ void lse_merge16(int ns, PartFn part, f16* out, int64_t out_hstride,
                                            float* lse) {
  auto ld1 = [](const float* p) { return kCoherent ? load_coherent(p) : *p; };
  auto ld4 = [](const float* p) { return kCoherent ? load_coherent4(p) : *(const f32x4*)p; };
  constexpr int kB = 8;   // splits per batch of LSE loads
  constexpr int kU = 2;   // splits per batch of output loads
  const int tid = threadIdx.x;
  const int n = tid >> 4;
  const int c0 = (tid & 15) * 32;
  float m = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += kB) {
    float v[kB];
#pragma unroll
    for (int j = 0; j < kB; j++) {
      const float* o;
      const float* l;
      if (s0 + j < ns) {
        part(s0 + j, &o, &l);
        v[j] = ld1(l + n);
      } else {
        v[j] = -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < kB; j++) m = fmaxf(m, v[j]);
  }
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; k++) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.0f;
  if (m != -INFINITY) {
    for (int s0 = 0; s0 < ns; s0 += kU) {
      float ls[kU];
      f32x4 ov[kU][8];
#pragma unroll
      for (int j = 0; j < kU; j++) {
        ls[j] = -INFINITY;
        if (s0 + j < ns) {
          const float* o;
          const float* l;
          part(s0 + j, &o, &l);
          ls[j] = ld1(l + n);
          const float* op = o + n * 512 + c0;
#pragma unroll
          for (int k = 0; k < 8; k++) ov[j][k] = ld4(op + 4 * k);
        }
      }
#pragma unroll
      for (int j = 0; j < kU; j++) {
        if (ls[j] == -INFINITY) continue;   // empty split (or past the end): weight 0
        const float e = expf(ls[j] - m);
        den += e;
#pragma unroll
        for (int k = 0; k < 8; k++) acc[k] += e * ov[j][k];
      }
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  f16* dst = out + (int64_t)n * out_hstride + c0;
#pragma unroll
  for (int k = 0; k < 8; k += 2) {
    const f32x4 a = acc[k] * inv, b = acc[k + 1] * inv;
    *(f16x8*)(dst + 4 * k) = f16x8{(f16)a.x, (f16)a.y, (f16)a.z, (f16)a.w,
                                   (f16)b.x, (f16)b.y, (f16)b.z, (f16)b.w};
  }
  if ((tid & 15) == 0) lse[n] = den > 0.0f ? m + logf(den) : -INFINITY;
}

}  // namespace smla

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
template <class PartFn>
__device__ __forceinline__ void lse_merge16(int ns, PartFn part, f16* out, int64_t out_hstride,
                                            float* lse) {
  const int tid = threadIdx.x;
  const int n = tid >> 4;            // head within the group
  const int c0 = (tid & 15) * 32;    // first of this thread's 32 columns
  float m = -INFINITY;
  for (int s = 0; s < ns; s++) {
    const float* o;
    const float* l;
    part(s, &o, &l);
    m = fmaxf(m, l[n]);
  }
  float den = 0.0f;
  if (m != -INFINITY) {
    for (int s = 0; s < ns; s++) {
      const float* o;
      const float* l;
      part(s, &o, &l);
      const float ls = l[n];
      if (ls != -INFINITY) den += expf(ls - m);
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  f16* dst = out + (int64_t)n * out_hstride + c0;
  for (int cb = 0; cb < 32; cb += 8) {   // 8 columns at a time keeps few registers live
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f}, b = f32x4{0.f, 0.f, 0.f, 0.f};
    if (den > 0.0f) {
      for (int s = 0; s < ns; s++) {
        const float* o;
        const float* l;
        part(s, &o, &l);
        const float ls = l[n];
        if (ls == -INFINITY) continue;
        const float e = expf(ls - m);
        const float* op = o + n * 512 + c0 + cb;
        a += e * *(const f32x4*)op;
        b += e * *(const f32x4*)(op + 4);
      }
    }
    a *= inv;
    b *= inv;
    *(f16x8*)(dst + cb) = f16x8{(f16)a.x, (f16)a.y, (f16)a.z, (f16)a.w,
                               (f16)b.x, (f16)b.y, (f16)b.z, (f16)b.w};
  }
  if ((tid & 15) == 0) lse[n] = den > 0.0f ? m + logf(den) : -INFINITY;
}

}  // namespace smla

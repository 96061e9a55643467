// Cache-row codec kernels for gfx950: the NVFP4 row writer (pack), the unpack export
// used by tests, pass 1 of the staged FP8 variant, and the 576-byte FP8 row writer.
//
// "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section
// "Four-bit caches make room": NVFP4 (one FP8 scale per 16 four-bit values) is the
// storage format of the MLA cache, 352 bytes per row; a staged implementation first
// unpacked NVFP4 values into FP8 buffers before attention.
#include "smla_device.hpp"
#include "smla_launch.hpp"

namespace smla {

// One wave per row.  Lanes 0..31 own latent group g = lane (16 values), lanes 32..63 own
// rope values 2r, 2r+1 (r = lane - 32).  The 352-byte row is assembled in LDS and written
// with 22 coalesced 16-byte stores, at the allocation row `map` gives for the slot (the
// slot itself in a layer-major pool).
__global__ __launch_bounds__(256) void nvfp4_pack_rows_kernel(const f16* __restrict__ src,
                                                               const int32_t* __restrict__ slots,
                                                               int32_t n, uint8_t* __restrict__ pool,
                                                               int64_t pool_rows, RowMap map) {
  __shared__ __attribute__((aligned(16))) uint8_t rowbuf[4][kRowBytes];
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wid;
  int32_t slot = -1;
  if (row < n) slot = slots[row];
  const bool active = slot >= 0 && (int64_t)slot < pool_rows;   // wave-uniform
  SMLA_LDS uint8_t* rb = (SMLA_LDS uint8_t*)rowbuf[wid];
  if (active) {
    const f16* x = src + row * kHeadDim;
    if (lane < 32) {
      const u32x4 v0 = *(const u32x4*)(x + 16 * lane);
      const u32x4 v1 = *(const u32x4*)(x + 16 * lane + 8);
      f16 h[16];
      __builtin_memcpy(&h[0], &v0, 16);
      __builtin_memcpy(&h[8], &v1, 16);
      float amax = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; k++) amax = fmaxf(amax, fabsf((float)h[k]));
      // E4M3 nearest to the exact real amax/6: a correctly rounded fp32 quotient never
      // crosses an E4M3 rounding boundary (an fp16 amax sits at least 2^-11 relative away
      // from 6 x any E4M3 midpoint unless exactly on it), so rounding it again is exact.
      const uint32_t sc = e4m3_encode_rne(__fdiv_rn(amax, 6.0f));
      const float s = (float)e4m3x2<false>(sc).x;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int k = 0; k < 8; k++) lo |= e2m1_encode((float)h[k], s) << (4 * k);
#pragma unroll
      for (int k = 0; k < 8; k++) hi |= e2m1_encode((float)h[8 + k], s) << (4 * k);
      lds_store<u32x2>(rb + 8 * lane, u32x2{lo, hi});
      rb[kScaleOff + lane] = (uint8_t)sc;
    } else {
      const int r = lane - 32;
      const f16x2 v = *(const f16x2*)(x + kLatent + 2 * r);
      const uint32_t c0 = e4m3_encode_rne((float)v.x), c1 = e4m3_encode_rne((float)v.y);
      lds_store<uint16_t>(rb + kRopeOff + 2 * r, (uint16_t)(c0 | (c1 << 8)));
    }
  }
  __syncthreads();
  if (active && lane < kRowBytes / 16) {
    const u32x4 v = lds_load<u32x4>(rb + 16 * lane);
    *(u32x4*)(pool + storage_row_wide((uint32_t)slot, map) * kRowBytes + 16 * lane) = v;
  }
}

// One wave per requested row: lane l decodes latent values 8l..8l+7 (one dword of codes,
// one group scale); lanes 0..7 also decode rope values 8l..8l+7.
__global__ __launch_bounds__(256) void nvfp4_unpack_rows_kernel(const uint8_t* __restrict__ pool,
                                                                 int64_t pool_rows,
                                                                 const int32_t* __restrict__ rows,
                                                                 int32_t n, f16* __restrict__ out) {
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + wid;
  if (i >= n) return;
  const int32_t r = rows[i];
  f16* o = out + i * kHeadDim;
  if (!row_valid(r, pool_rows)) {
    *(u32x4*)(o + 8 * lane) = u32x4{0, 0, 0, 0};
    if (lane < 8) *(u32x4*)(o + kLatent + 8 * lane) = u32x4{0, 0, 0, 0};
    return;
  }
  const uint8_t* p = pool + (int64_t)r * kRowBytes;
  const uint32_t w = *(const uint32_t*)(p + 4 * lane);
  const uint32_t sc = p[kScaleOff + lane / 2];
  const f16 s = e4m3x2<false>(sc).x;
  const f16x8 v = unpack8(w, f16x2{s, s});
  *(f16x8*)(o + 8 * lane) = v;
  if (lane < 8) {
    const u32x2 rp = *(const u32x2*)(p + kRopeOff + 8 * lane);
    *(f16x8*)(o + kLatent + 8 * lane) = fp8x8(rp.x, rp.y);
  }
}

// Staged pass 1: sixteen lanes per list entry, four entries per wave, kStageRounds rounds of
// entries per wave with every load of a round issued before any conversion.  Lane l of an
// entry re-encodes latent groups l and 16 + l (two 8-byte code loads, two scale bytes) and
// writes them as 16-byte stores at offsets 16l and 256 + 16l, so each store instruction
// fills 256 contiguous bytes of the entry's output row; lanes 0..3 copy the rope (already
// E4M3).  Empty entries write zeros.  The output is written with non-temporal stores: it
// exceeds the caches and is read back only by the attention pass.
constexpr int kStageRounds = 4;

__global__ __launch_bounds__(256) void nvfp4_stage_fp8_kernel(const uint8_t* __restrict__ pool,
                                                              int64_t pool_rows,
                                                              const int32_t* __restrict__ idx,
                                                              int64_t entries,
                                                              uint8_t* __restrict__ staged) {
  const int q = threadIdx.x >> 4, l = threadIdx.x & 15;
  const int64_t e0 = (int64_t)blockIdx.x * (16 * kStageRounds) + q;
  uint32_t code[kStageRounds][4], sc[kStageRounds][2];
  u32x4 rope[kStageRounds];
  bool ok[kStageRounds];
#pragma unroll
  for (int u = 0; u < kStageRounds; u++) {
    const int64_t e = e0 + 16 * u;
    const int32_t r = e < entries ? idx[e] : -1;
    ok[u] = row_valid(r, pool_rows);
    code[u][0] = code[u][1] = code[u][2] = code[u][3] = 0;
    sc[u][0] = sc[u][1] = 0;
    rope[u] = u32x4{0, 0, 0, 0};
    if (ok[u]) {
      const uint8_t* p = pool + (int64_t)r * kRowBytes;
      const u32x2 a = *(const u32x2*)(p + 8 * l);
      const u32x2 b = *(const u32x2*)(p + 128 + 8 * l);
      code[u][0] = a.x;
      code[u][1] = a.y;
      code[u][2] = b.x;
      code[u][3] = b.y;
      sc[u][0] = p[kScaleOff + l];
      sc[u][1] = p[kScaleOff + 16 + l];
      if (l < 4) rope[u] = *(const u32x4*)(p + kRopeOff + 16 * l);
    }
  }
#pragma unroll
  for (int u = 0; u < kStageRounds; u++) {
    const int64_t e = e0 + 16 * u;
    if (e >= entries) break;
    uint8_t* o = staged + e * kHeadDim;
    u32x4 v[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const f16 s = e4m3x2<false>(sc[u][h]).x;
      const f16x8 lo = unpack8(code[u][2 * h], f16x2{s, s});
      const f16x8 hi = unpack8(code[u][2 * h + 1], f16x2{s, s});
      const u32x2 a = e4m3x8_sat(lo), b = e4m3x8_sat(hi);
      v[h] = u32x4{a.x, a.y, b.x, b.y};
    }
    __builtin_nontemporal_store(v[0], (u32x4*)(o + 16 * l));
    __builtin_nontemporal_store(v[1], (u32x4*)(o + 256 + 16 * l));
    if (l < 4) __builtin_nontemporal_store(rope[u], (u32x4*)(o + kLatent + 16 * l));
  }
}

// The 576-byte FP8 cache row (the format NVFP4 replaces in "Four-bit caches make room"):
// byte k is the E4M3 code of value k.  One wave per row; lane l encodes the 8 values of
// piece l (and lanes 0..7 also piece 64 + l, the rope part) and writes them as 8 bytes.
__global__ __launch_bounds__(256) void fp8_pack_rows_kernel(const f16* __restrict__ src,
                                                             const int32_t* __restrict__ slots, int32_t n,
                                                             uint8_t* __restrict__ pool, int64_t pool_rows) {
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wid;
  if (row >= n) return;
  const int32_t slot = slots[row];
  if (slot < 0 || (int64_t)slot >= pool_rows) return;
  const f16* x = src + row * kHeadDim;
  uint8_t* o = pool + (int64_t)slot * kHeadDim;
  for (int p = lane; p < kHeadDim / 8; p += 64) {
    const u32x4 v = *(const u32x4*)(x + 8 * p);
    f16 h[8];
    __builtin_memcpy(h, &v, 16);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      lo |= e4m3_encode_rne((float)h[k]) << (8 * k);
      hi |= e4m3_encode_rne((float)h[4 + k]) << (8 * k);
    }
    *(u32x2*)(o + 8 * p) = u32x2{lo, hi};
  }
}

hipError_t launch_fp8_pack(const void* src, const int32_t* slots, int32_t n, void* pool, int64_t pool_rows,
                           hipStream_t s) {
  const int blocks = (n + 3) / 4;
  hipLaunchKernelGGL(fp8_pack_rows_kernel, dim3(blocks), dim3(256), 0, s, (const f16*)src, slots, n,
                     (uint8_t*)pool, pool_rows);
  return hipGetLastError();
}

hipError_t launch_pack(const void* src, const int32_t* slots, int32_t n, void* pool,
                       int64_t pool_rows, const RowMap& map, hipStream_t s) {
  const int blocks = (n + 3) / 4;
  hipLaunchKernelGGL(nvfp4_pack_rows_kernel, dim3(blocks), dim3(256), 0, s, (const f16*)src, slots,
                     n, (uint8_t*)pool, pool_rows, map);
  return hipGetLastError();
}

hipError_t launch_unpack(const void* pool, int64_t pool_rows, const int32_t* rows, int32_t n,
                         void* out, hipStream_t s) {
  const int blocks = (n + 3) / 4;
  hipLaunchKernelGGL(nvfp4_unpack_rows_kernel, dim3(blocks), dim3(256), 0, s,
                     (const uint8_t*)pool, pool_rows, rows, n, (f16*)out);
  return hipGetLastError();
}

hipError_t launch_stage_fp8(const void* pool, int64_t pool_rows, const int32_t* idx,
                            int64_t entries, void* staged, hipStream_t s) {
  const int64_t blocks = (entries + 16 * kStageRounds - 1) / (16 * kStageRounds);
  hipLaunchKernelGGL(nvfp4_stage_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const uint8_t*)pool, pool_rows, idx, entries, (uint8_t*)staged);
  return hipGetLastError();
}

}  // namespace smla

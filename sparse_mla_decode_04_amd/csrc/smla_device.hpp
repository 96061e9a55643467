// Device-side building blocks shared by the gfx950 kernels: vector types, the exact
// FP8 E4M3 / E2M1 encoders of the cache-row writer, the on-chip NVFP4 unpack, MFMA and
// LDS transpose-read wrappers.
//
// Row format ("Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily",
// section "Four-bit caches make room": NVFP4 with one FP8 scale per 16 values, 352-byte
// rows): [0,256) E2M1 codes (even element in the low nibble), [256,288) E4M3 group
// scales, [288,352) E4M3 rope values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

#define SMLA_LDS __attribute__((address_space(3)))

constexpr int kRowBytes = 352;
constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kHeadDim = 576;
constexpr int kScaleOff = 256;
constexpr int kRopeOff = 288;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ bool row_valid(int32_t r, int64_t pool_rows) {
  return r >= 0 && (int64_t)r < pool_rows;
}

// ------------------------------------------------------------------ encoders -----
// Nearest FP8 E4M3 ("FN": bias 7, max 448, no infinities) code of a finite float,
// ties to the even code, saturating at +-448, sign kept.  Exact: the power-of-two
// rescalings are exact and rintf rounds half to even.
__device__ __forceinline__ uint32_t e4m3_encode_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid m * 2^-9
    code = (uint32_t)rintf(a * 512.0f);      // 0..8; 8 is the smallest normal (0x08)
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // a in [2^e, 2^(e+1))
    float r = rintf(ldexpf(a, 3 - e));       // in [8, 16]
    if (r == 16.0f) { e += 1; r = 8.0f; }
    code = ((uint32_t)(e + 7) << 3) | ((uint32_t)r - 8u);
  }
  return sign | code;
}

// Nearest E2M1 code of the exact real x/s (s = a decoded E4M3 scale, >= 0), ties to the
// even code, saturating at 6, sign kept; s == 0 gives the signed zero.  Division-free:
// |x| is compared with s times the midpoints of the E2M1 grid {0,.5,1,1.5,2,3,4,6};
// those products have at most 7 significant bits and are exact in fp32.  An exact tie
// goes to the even code: up at 0.75, 1.75 and 3.5 (the upper neighbour's code is even),
// down at 0.25, 1.25, 2.5 and 5 (the lower neighbour's code is even).
__device__ __forceinline__ uint32_t e2m1_encode(float x, float s) {
  const float m = fabsf(x);
  uint32_t c = 0;
  if (s > 0.0f) {
    c = (uint32_t)(m > 0.25f * s) + (uint32_t)(m >= 0.75f * s) + (uint32_t)(m > 1.25f * s) +
        (uint32_t)(m >= 1.75f * s) + (uint32_t)(m > 2.5f * s) + (uint32_t)(m >= 3.5f * s) +
        (uint32_t)(m > 5.0f * s);
  }
  return c | ((__float_as_uint(x) >> 28) & 0x8u);
}

// ------------------------------------------------------------------ decoders -----
// Two E2M1 codes (byte SEL of w) -> two fp16, unscaled.  The gfx950 scaled convert only
// honours the exponent of its scale operand, so it is used with scale 1 and the E4M3
// group scale is applied by an exact fp16 multiply (an E2M1 x E4M3 product has at most
// 6 significant bits and lies within fp16's normal/subnormal range).
template <int SEL>
__device__ __forceinline__ f16x2 e2m1x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
// Two E4M3 codes (low or high 16 bits of w) -> two fp16 (exact).
template <bool HI>
__device__ __forceinline__ f16x2 e4m3x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Eight consecutive latent values (one dword of codes) times one group scale.
__device__ __forceinline__ f16x8 unpack8(uint32_t w, f16x2 ss) {
  f16x2 a = e2m1x2<0>(w) * ss, b = e2m1x2<1>(w) * ss, c = e2m1x2<2>(w) * ss, d = e2m1x2<3>(w) * ss;
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}
// Eight codes of one dword where value pair j uses its own scale pair sc[j].
__device__ __forceinline__ f16x8 unpack8_pairs(uint32_t w, f16x8 sc) {
  f16x2 a = e2m1x2<0>(w) * f16x2{sc[0], sc[1]};
  f16x2 b = e2m1x2<1>(w) * f16x2{sc[2], sc[3]};
  f16x2 c = e2m1x2<2>(w) * f16x2{sc[4], sc[5]};
  f16x2 d = e2m1x2<3>(w) * f16x2{sc[6], sc[7]};
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}
// Eight E4M3 codes (two dwords) -> eight fp16.
__device__ __forceinline__ f16x8 fp8x8(uint32_t lo, uint32_t hi) {
  f16x2 a = e4m3x2<false>(lo), b = e4m3x2<true>(lo), c = e4m3x2<false>(hi), d = e4m3x2<true>(hi);
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Four fp16 values -> four E4M3 codes in one dword (value k in byte k): nearest, ties to
// the even code, saturating at +-448, sign kept.  The gfx950 conversion (scale 1) rounds
// to nearest even; clamping to the largest finite E4M3 magnitude first gives the
// saturation, since no clamped value lies past 448.
__device__ __forceinline__ uint32_t e4m3x4_sat(f16x2 a, f16x2 b) {
  const f16x2 lo = f16x2{(f16)-448.0f, (f16)-448.0f}, hi = f16x2{(f16)448.0f, (f16)448.0f};
  a = __builtin_elementwise_min(__builtin_elementwise_max(a, lo), hi);
  b = __builtin_elementwise_min(__builtin_elementwise_max(b, lo), hi);
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  s16x2 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, a, 1.0f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, b, 1.0f, true);
  return __builtin_bit_cast(uint32_t, r);
}
// Eight fp16 values -> eight E4M3 codes in two dwords (as e4m3x4_sat).
__device__ __forceinline__ u32x2 e4m3x8_sat(f16x8 v) {
  return u32x2{e4m3x4_sat(f16x2{v[0], v[1]}, f16x2{v[2], v[3]}), e4m3x4_sat(f16x2{v[4], v[5]}, f16x2{v[6], v[7]})};
}

// ------------------------------------------------------------------ matrix cores --
// D = A(16x32) * B(32x16) + C with fp16 operands and fp32 accumulation.  Lane l holds
// A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16], and C/D[4*(l/16) .. +3][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// D = A(32x16) * B(16x32) + C.  Lane l holds A[l%32][8*(l/32) .. +7], B[8*(l/32) .. +7][l%32],
// and element i of C/D is [8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// LDS transpose read of 4-bit elements: within each group of 16 lanes, lane s supplies
// the address of 8 bytes (16 nibbles); lane i receives nibble i of every lane s of its
// group, lane s's nibble landing at nibble position s of the result.
__device__ __forceinline__ u32x2 lds_read_tr4(const SMLA_LDS void* p) {
  i32x2 v = __builtin_amdgcn_ds_read_tr4_b64_v2i32((SMLA_LDS i32x2*)p);
  return u32x2{(uint32_t)v.x, (uint32_t)v.y};
}

// LDS transpose read of 8-bit elements: within each group of 16 lanes, the 8-byte chunks
// the lanes address, in lane order, form a row-major 8 x 16 byte matrix (lanes 2r and
// 2r+1 make row r); lane i receives column i, row r in byte r.
__device__ __forceinline__ u32x2 lds_read_tr8(const SMLA_LDS void* p) {
  i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SMLA_LDS i32x2*)p);
  return u32x2{(uint32_t)v.x, (uint32_t)v.y};
}

// LDS loads / stores through an LDS-qualified pointer, or through a generic pointer to a
// __shared__ object (cast to the LDS address space so the compiler emits ds_* ops).
template <typename T>
__device__ __forceinline__ T lds_load(const SMLA_LDS void* p) {
  return *(const SMLA_LDS T*)p;
}
template <typename T>
__device__ __forceinline__ void lds_store(SMLA_LDS void* p, T v) {
  *(SMLA_LDS T*)p = v;
}
template <typename T>
__device__ __forceinline__ T lds_load(const void* p) {
  return *(const SMLA_LDS T*)p;
}
template <typename T>
__device__ __forceinline__ void lds_store(void* p, T v) {
  *(SMLA_LDS T*)p = v;
}

// Reductions over the four lanes l, l^16, l^32, l^48 with the gfx950 lane-swap
// instructions (no LDS round trip).  permlane16_swap(v, v) yields, in every lane, the
// values of its even and its odd 16-lane row; permlane32_swap(v, v) those of its lower and
// upper 32-lane half.  Every lane of a quadruple combines the same operands in the same
// order, so all four get bit-identical results.
__device__ __forceinline__ float wave_max_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Maximum over lanes l and l^32.
__device__ __forceinline__ float wave_max_xor32(float v) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace smla

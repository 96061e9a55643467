// Pieces shared by the two sparse MLA decode kernels (LDS-ring gather in decode.hip,
// register-pipelined gather in decode_regs.hip): tile cursor, query registers, the
// end-of-segment write (output or split partial) and the in-launch merge of a token's
// partials.
//
// "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section
// "Four-bit caches make room": attention over the rows the index list names, FP16
// operands, FP32 accumulation, work decomposition sized by the token batch.
#pragma once

#include "smla_combine.hpp"
#include "smla_decode.hpp"
#include "smla_device.hpp"

namespace smla {

constexpr int kWaves = 4;               // waves per workgroup
constexpr int kWR = 16;                 // tile rows per wave
constexpr int kPH = 72;                 // fp16 stride of the [.][tile row] LDS tables
constexpr float kSlack = 8.0f;          // log2 units a wave may exceed the shared reference by
constexpr uint32_t kOOB = 0xFFFFF000u;  // buffer offset beyond every range (reads as zero),
                                        // also with an instruction offset of up to 4095 added:
                                        // every buffer the kernels address is at most kOOB bytes

// Tile cursor: flat tile c -> token t and tile ci within the token, advanced one at a time.
// The tile count of a launch is below 2^31 (checked on the host).
struct Cursor {
  int32_t c;
  int32_t t;
  int32_t ci;
  __device__ void init(int64_t c0, int32_t cpt) {
    c = (int32_t)c0;
    t = c / cpt;
    ci = c - t * cpt;
  }
  __device__ void next(int32_t cpt) {
    c++;
    if (++ci == cpt) {
      ci = 0;
      t++;
    }
  }
};

// B operands of the QK^T steps for lane (head r16, k-group g): step k < 16 covers latent
// features 128g + 8k .. +7, steps 16 and 17 the rope features 512 + 16g .. +15.
template <int NG>
struct QReg {
  f16x8 v[NG][18];
};

template <int NG>
__device__ __forceinline__ void load_q(const DecodeArgs& A, int64_t t, int head0, int r16, int g,
                                       QReg<NG>& Q) {
#pragma unroll
  for (int j = 0; j < NG; j++) {
    const f16* base = (const f16*)A.q + ((t * A.H + head0 + kHeadGroup * j + r16) * kHeadDim);
#pragma unroll
    for (int k = 0; k < 16; k++) Q.v[j][k] = *(const f16x8*)(base + 128 * g + 8 * k);
    Q.v[j][16] = *(const f16x8*)(base + kLatent + 16 * g);
    Q.v[j][17] = *(const f16x8*)(base + kLatent + 16 * g + 8);
  }
}

// The LDS DMA sequences below set m0 themselves and declare it clobbered.
#pragma clang diagnostic ignored "-Winline-asm"

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): raw byte addressing; an offset at or past
// `bytes` reads as zero without a memory access.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;   // 32-bit data format, no swizzle
  return r;
}

// LDS DMA: lane l's 16 (4) bytes at buffer offset voff land at LDS byte lds + 16*l (4*l).
// Issued as inline assembly so the compiler neither waits for nor reorders around them
// implicitly; every consumer waits with an explicit vmcnt.
__device__ __forceinline__ void dma16(i32x4 rs, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rs)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(i32x4 rs, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rs)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N): vector memory operations complete in issue order, so this waits
// for everything but the N most recent.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS byte address of p (wave-uniform: DMA destinations go through m0).
__device__ __forceinline__ uint32_t lds_addr(const SMLA_LDS void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// Query staging: the 16*NG query rows of a token (1152 bytes each) as 16-byte pieces with
// one spare piece per row (row stride 1168 bytes keeps the register loads conflict-free),
// filled by kLoads DMA instructions of 1 KB.
template <int NG>
struct QFmt {
  static constexpr int kSlots = kHeadGroup * NG * 73;        // 72 pieces + 1 spare per head
  static constexpr int kLoads = (kSlots + 63) / 64;          // 19 or 37
  static constexpr int kBytes = kLoads * 1024;
};

// DMA of wave wid's share (instructions wid, wid+4, ...) of the query rows of token t of
// heads head0 .. head0+16*NG-1 into the staging area at LDS byte lds0.
template <int NG>
__device__ __forceinline__ void dma_q(const DecodeArgs& A, i32x4 rs_q, int64_t t, int head0, int wid, int lane,
                                      uint32_t lds0) {
  constexpr int NH = kHeadGroup * NG;
  constexpr int kPerWave = (QFmt<NG>::kLoads + kWaves - 1) / kWaves;
#pragma unroll
  for (int u = 0; u < kPerWave; u++) {
    const int kk = wid + kWaves * u;
    if (kk >= QFmt<NG>::kLoads) break;
    const int sl = 64 * kk + lane, h = sl / 73, p = sl - 73 * h;
    const bool ok = h < NH && p < 72;
    const uint32_t voff = ok ? (uint32_t)((t * A.H + head0 + h) * (int64_t)(2 * kHeadDim)) + 16u * p : kOOB;
    dma16(rs_q, voff, lds0 + 1024u * kk);
  }
}

// Query registers from the staging area (layout of QFmt).
template <int NG>
__device__ __forceinline__ void read_q(const SMLA_LDS uint8_t* qs, int r16, int g, QReg<NG>& Q) {
#pragma unroll
  for (int j = 0; j < NG; j++) {
    const SMLA_LDS uint8_t* h = qs + (kHeadGroup * j + r16) * 1168;
#pragma unroll
    for (int k = 0; k < 16; k++) Q.v[j][k] = lds_load<f16x8>(h + 16 * (16 * g + k));
    Q.v[j][16] = lds_load<f16x8>(h + 16 * (64 + 2 * g));
    Q.v[j][17] = lds_load<f16x8>(h + 16 * (65 + 2 * g));
  }
}

// Sum of eight fp16 values in fp32.
__device__ __forceinline__ float sum8(f16x8 v) {
  const f16x2 one = f16x2{(f16)1.0f, (f16)1.0f};
  float s = __builtin_amdgcn_fdot2(f16x2{v[0], v[1]}, one, 0.0f, false);
  s = __builtin_amdgcn_fdot2(f16x2{v[2], v[3]}, one, s, false);
  s = __builtin_amdgcn_fdot2(f16x2{v[4], v[5]}, one, s, false);
  return __builtin_amdgcn_fdot2(f16x2{v[6], v[7]}, one, s, false);
}

// End of a token segment of a range.  O[j][k] holds O^T for features 16*(8*wid + k) +
// 4g .. +3 of head 16j + r16 (unnormalized, base-2 reference m_ref, denominator l_acc
// summed over the lane's rows).  A range that covers the whole token writes out and lse;
// otherwise it writes its normalized partial and natural-log LSE into partial slot
// slot_id with device-coherent stores.  The state is reset for the next segment.
template <int NG>
__device__ __forceinline__ void finish_segment(const DecodeArgs& A, f32x4 (&O)[NG][8], float (&m_ref)[NG],
                                               float (&l_acc)[NG], int64_t t, bool full, int64_t slot_id,
                                               int head0, int wid, int g, int r16,
                                               __amdgpu_buffer_rsrc_t ws_o, __amdgpu_buffer_rsrc_t ws_l) {
  constexpr int NH = kHeadGroup * NG;
#pragma unroll
  for (int j = 0; j < NG; j++) {
    const float Ls = wave_sum_xor16_32(l_acc[j]);
    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
    const float lse_nat = Ls > 0.0f ? (m_ref[j] + log2f(Ls)) * kLn2 : -INFINITY;
    const int hl = kHeadGroup * j + r16;   // head within the block
    if (full) {
      f16* op = (f16*)A.out + (t * A.H + head0 + hl) * kLatent;
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const f32x4 v = O[j][k] * inv;
        *(f16x4*)(op + 16 * (8 * wid + k) + 4 * g) = f16x4{(f16)v.x, (f16)v.y, (f16)v.z, (f16)v.w};
      }
      if (wid == 0 && g == 0) A.lse[t * A.H + head0 + hl] = lse_nat;
    } else {
      const uint32_t po = (uint32_t)((slot_id * NH + hl) * kLatent) * 4u;
#pragma unroll
      for (int k = 0; k < 8; k++) merge_st4(ws_o, po + 4u * (16 * (8 * wid + k) + 4 * g), O[j][k] * inv);
      if (wid == 0 && g == 0) merge_st1(ws_l, (uint32_t)(slot_id * NH + hl) * 4u, lse_nat);
    }
#pragma unroll
    for (int k = 0; k < 8; k++) O[j][k] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref[j] = -INFINITY;
    l_acc[j] = 0.0f;
  }
}

// After a range's last tile: publish its partials (every store of the workgroup complete,
// then one counter increment per pending token) and, for each token whose last range this
// is, merge the token's partials into out / lse.  pend_t[seg] is the token this range wrote
// partial slot seg for, or -1.  flag: one int of LDS; scratch: >= 2048 floats of idle LDS.
// Bit seg of `counted`: the range counted itself for token pend_t[seg] earlier and found it
// was the last (pend_t[seg] is -1 if it was not): merge without counting again.
template <int NH>
__device__ __forceinline__ void publish_and_merge(const DecodeArgs& A, const int64_t (&pend_t)[2], int hb, int head0,
                                                  __amdgpu_buffer_rsrc_t ws_o,
                                                  __amdgpu_buffer_rsrc_t ws_l, int* flag, float* scratch,
                                                  int counted = 0) {
  const int64_t C = A.tiles;
  const int G = A.G;
  const int cpt = A.cpt;
  const int tid = threadIdx.x;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int seg = 0; seg < 2; seg++) {
    const int64_t t = pend_t[seg];
    if (t < 0) continue;
    const int64_t tok0 = t * cpt;
    const int64_t w_lo = wg_of_chunk(tok0, C, G), w_hi = wg_of_chunk(tok0 + cpt - 1, C, G);
    if (tid == 0) {
      int last = 1;
      if (!((counted >> seg) & 1)) {
        int32_t* cnt = A.counters + (int64_t)hb * A.T + t;
        const int old = atomicAdd(cnt, 1);
        last = (old == (int)(w_hi - w_lo));
        if (last) atomicExch(cnt, 0);
      }
      *flag = last;
    }
    __syncthreads();
    const int last = *flag;
    __syncthreads();
    if (!last) continue;
    // split s of token t is range w_lo + s.  Every range after w_lo starts inside the
    // token, so t is its first token (slot 0); range w_lo holds t in slot 1 exactly when
    // it starts before the token.
    const uint32_t sl0 = (uint32_t)(((int64_t)hb * G + w_lo) * 2);
    const uint32_t seg0 = (wg_first_chunk(w_lo, C, G) < tok0) ? 1u : 0u;
    auto part = [&](int s, uint32_t* o_off, uint32_t* l_off) {
      const uint32_t sl = sl0 + 2u * (uint32_t)s + (s == 0 ? seg0 : 0u);
      *o_off = sl * (uint32_t)(NH * kLatent * 4);
      *l_off = sl * (uint32_t)(NH * 4);
    };
    lse_merge<NH, true>((int)(w_hi - w_lo + 1), ws_o, ws_l, part,
                        (f16*)A.out + (t * A.H + head0) * kLatent, A.lse + t * A.H + head0, scratch, tid);
    __syncthreads();
  }
}

}  // namespace smla

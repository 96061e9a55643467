// Fused sparse MLA decode over NVFP4 cache rows for gfx950 (MI355X).
//
// "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section
// "Four-bit caches make room": for every decode token the kernel loads only the cache
// rows named by the sparse indexer's 2,048-entry list, unpacks the NVFP4 values on chip
// (no FP8 staging buffer in HBM), and runs attention with FP16 operands and FP32
// accumulation; empty list entries cost no load.  The page's kernel overlaps unpacking
// with scoring/accumulation through a three-slot pipeline over warp groups and sizes
// SM clusters by the token batch; the gfx950 design below keeps the overlap and the
// batch-sized decomposition but maps them onto wave64 / MFMA / LDS:
//
//  * Workgroup = 4 waves, one 16-head group, a contiguous range of 64-row chunks of the
//    flattened (token, chunk) sequence (stream-K split, see smla_decode.hpp).  Block ids
//    are remapped so that consecutive ranges -- which share tokens -- run on one XCD.
//  * Gather: each wave fetches its 16 rows of a chunk with coalesced 16-byte loads
//    (22 per 352-byte row) into registers two chunks ahead, and stores them into a
//    double-buffered LDS slot one chunk ahead.  Empty entries issue no load and store
//    zeros.  Several waves per SIMD keep MFMA, VALU unpack and loads in flight at once.
//  * QK^T: wave w scores rows 16w..16w+15 of the chunk against the 16 heads with
//    v_mfma_f32_16x16x32_f16 (M = rows, N = heads, K = 576 in 18 steps).  Each lane
//    unpacks its own row's codes straight into the A operand (E2M1 -> fp16 by the
//    hardware convert, times the E4M3 group scale by an exact fp16 multiply); the query
//    tile stays in registers as the B operand.
//  * Online softmax in fp32 (base-2, scores pre-scaled by softmax_scale*log2 e), with a
//    shared running maximum that is only raised when a chunk's maximum exceeds it by
//    more than 8 (so rescaling of the accumulator is rare and probabilities stay <= 256
//    in fp16).  Empty entries get probability 0.
//  * PV: wave w owns output features 128w..128w+127 (8 tiles of 16 = one scale group
//    each) for all 16 heads and all 64 rows: O^T += V^T P^T with M = features, N = heads,
//    K = rows.  The V^T operand comes straight from the raw nibbles through the LDS
//    4-bit transpose read (ds_read_b64_tr_b4: 16 rows of one feature per lane), scaled
//    by a per-chunk fp16 table of the rows' E4M3 scales (zero for empty rows); P^T is
//    exchanged through LDS.
//  * Epilogue: a workgroup that owns a whole token writes out = O/l and lse directly;
//    otherwise it writes its normalized partial and LSE, and the last workgroup of the
//    token (device-scope counter) merges the partials (smla_combine.hpp).
//
// The same skeleton, instantiated with kFp8 = true, is pass 2 of the staged variant: it
// attends over 576-byte FP8 E4M3 rows written to HBM by pass 1 (one per list entry),
// reading V^T through the 8-bit LDS transpose read instead of the 4-bit one.
#include "smla_combine.hpp"
#include "smla_device.hpp"
#include "smla_launch.hpp"

namespace smla {

namespace {

constexpr int kWaves = 4;
constexpr int kWaveRows = 16;                               // rows gathered/scored per wave
constexpr int kPad = 72;                                   // fp16 row stride of sc/pb tables
constexpr float kRescaleSlack = 8.0f;                      // log2 units
constexpr int kQStride = kHeadDim + 8;                     // fp16 stride of the LDS query tile
constexpr int kQPieces = kHeadGroup * kHeadDim * 2 / 16;   // 1152 16-byte pieces per tile
constexpr int kQLoads = (kQPieces + 255) / 256;            // 5 per thread

template <bool kFp8>
struct Fmt {
  static constexpr int kRB = kFp8 ? kHeadDim : kRowBytes;          // bytes per row
  static constexpr int kPiecesPerRow = kRB / 16;                   // 22 or 36
  static constexpr int kWavePieces = kWaveRows * kPiecesPerRow;    // 352 or 576
  static constexpr int kLoads = (kWavePieces + 63) / 64;           // 6 or 9 per lane
  static constexpr int kSlotBytes = kChunkRows * kRB;
};

template <bool kFp8>
struct __attribute__((aligned(16))) Smem {
  uint8_t ring[2][Fmt<kFp8>::kSlotBytes];   // raw rows of the chunk being scored / the next
  f16 sc[kFp8 ? 1 : 32][kPad];              // [scale group][row] fp16 scales, 0 for empty rows
  f16 pb[kHeadGroup][kPad];                 // [head][row] fp16 probabilities
  f16 qs[kHeadGroup][kQStride];             // query tile of the current token, [head][576]
  float xmax[kWaves][kHeadGroup];           // per-wave chunk maxima
  float lsum[kWaves][kHeadGroup];           // per-wave softmax denominators
  int flag;
};

template <bool kFp8>
struct Stage {
  u32x4 v[Fmt<kFp8>::kLoads];
  int32_t idx;   // lane < 16: pool row of wave row `lane` (or -1)
};

__device__ __forceinline__ int32_t load_idx(const DecodeArgs& A, int64_t c, int wid, int lane) {
  const int64_t t = c / A.cpt;
  const int k = (int)(c - t * A.cpt) * kChunkRows + kWaveRows * wid + lane;
  int32_t v = -1;
  if (lane < kWaveRows && k < A.topk) v = A.idx[t * A.topk + k];
  return v;
}

// Fetch this wave's 16 rows of chunk c into registers.  NVFP4 rows come from the pool at
// their list index; FP8 rows (staged variant) sit at their list position.
template <bool kFp8>
__device__ __forceinline__ void issue(const DecodeArgs& A, int64_t c, int32_t idxv, Stage<kFp8>& S,
                                      int wid, int lane) {
  using F = Fmt<kFp8>;
  S.idx = idxv;
  const uint8_t* src = (const uint8_t*)A.rows;
  const int64_t t = c / A.cpt;
  const int64_t entry0 = t * A.topk + (c - t * A.cpt) * kChunkRows + kWaveRows * wid;
#pragma unroll
  for (int k = 0; k < F::kLoads; k++) {
    const int p = 64 * k + lane;
    const int r = p / F::kPiecesPerRow;                 // wave row of this piece
    const int off = (p - F::kPiecesPerRow * r) * 16;
    const int32_t row = __shfl(idxv, r & 15);
    u32x4 v = u32x4{0, 0, 0, 0};
    if (p < F::kWavePieces && row_valid(row, A.pool_rows)) {
      const int64_t base = kFp8 ? (entry0 + r) * (int64_t)kHeadDim : (int64_t)row * kRowBytes;
      v = *(const u32x4*)(src + base + off);
    }
    S.v[k] = v;
  }
}

template <bool kFp8>
__device__ __forceinline__ void commit(const Stage<kFp8>& S, SMLA_LDS uint8_t* slot, int wid, int lane) {
  using F = Fmt<kFp8>;
  SMLA_LDS uint8_t* base = slot + wid * (kWaveRows * F::kRB);
#pragma unroll
  for (int k = 0; k < F::kLoads; k++) {
    const int p = 64 * k + lane;
    if (p < F::kWavePieces) lds_store<u32x4>(base + 16 * p, S.v[k]);
  }
}

template <bool kFp8>
__device__ __forceinline__ uint64_t valid_mask(const DecodeArgs& A, const Stage<kFp8>& S, int lane) {
  return __ballot(lane < kWaveRows && row_valid(S.idx, A.pool_rows));
}

__device__ __forceinline__ u32x2 lds_read_tr8(const SMLA_LDS void* p) {
  i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SMLA_LDS i32x2*)p);
  return u32x2{(uint32_t)v.x, (uint32_t)v.y};
}

// Query tile of token t for head group hg: 16 heads x 576 fp16, fetched by the whole
// workgroup (thread tid takes pieces tid, tid+256, ...).
struct QStage {
  u32x4 v[kQLoads];
};

__device__ __forceinline__ void issue_q(const DecodeArgs& A, int64_t t, int hg, QStage& Q) {
  const int tid = threadIdx.x;
  const uint8_t* base = (const uint8_t*)A.q + ((t * A.H + (int64_t)kHeadGroup * hg) * kHeadDim) * 2;
#pragma unroll
  for (int k = 0; k < kQLoads; k++) {
    const int p = 256 * k + tid;
    u32x4 v = u32x4{0, 0, 0, 0};
    if (p < kQPieces) v = *(const u32x4*)(base + 16 * p);   // heads are contiguous in q
    Q.v[k] = v;
  }
}

__device__ __forceinline__ void commit_q(const QStage& Q, f16 (*qs)[kQStride]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < kQLoads; k++) {
    const int p = 256 * k + tid;
    if (p < kQPieces) {
      const int h = p / (kHeadDim * 2 / 16), off = (p - h * (kHeadDim * 2 / 16)) * 8;
      lds_store<u32x4>(&qs[h][off], Q.v[k]);
    }
  }
}

}  // namespace

template <bool kFp8>
__global__ __launch_bounds__(256, kFp8 ? 1 : 2) void sparse_mla_decode_kernel(DecodeArgs A) {
  using F = Fmt<kFp8>;
  __shared__ Smem<kFp8> sm;
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int hg = blockIdx.y;
  const int G = A.G;
  // XCD-aware order: hardware deals block b to XCD b % 8; give each XCD a contiguous
  // run of logical workgroups so that neighbouring ranges (same tokens) share an L2.
  const int bx = blockIdx.x, xcd = bx & 7, G8 = G >> 3, Gr = G & 7;
  const int w = xcd * G8 + min(xcd, Gr) + (bx >> 3);
  const int64_t C = A.chunks;
  const int64_t c_lo = wg_first_chunk(w, C, G), c_hi = wg_first_chunk(w + 1, C, G);
  const int n = (int)(c_hi - c_lo);
  const int cpt = A.cpt;

  SMLA_LDS uint8_t* ring0 = (SMLA_LDS uint8_t*)sm.ring[0];
  SMLA_LDS uint8_t* ring1 = (SMLA_LDS uint8_t*)sm.ring[1];

  // ---- prologue: chunks 0 and 1 in flight, chunk 0 in LDS
  // Index lists run two chunks ahead of the row loads: loads complete in issue order, so
  // waiting for an index load also waits for every load issued before it.
  Stage<kFp8> s0, s1;
  const int32_t idx0 = load_idx(A, c_lo, wid, lane);
  const int32_t idx1 = (n > 1) ? load_idx(A, c_lo + 1, wid, lane) : -1;
  int32_t idx_a = (n > 2) ? load_idx(A, c_lo + 2, wid, lane) : -1;   // chunk i+2 at step i
  int32_t idx_b = (n > 3) ? load_idx(A, c_lo + 3, wid, lane) : -1;   // chunk i+3 at step i
  issue(A, c_lo, idx0, s0, wid, lane);
  if (n > 1) issue(A, c_lo + 1, idx1, s1, wid, lane);
  QStage qst;
  issue_q(A, c_lo / cpt, hg, qst);
  uint64_t vm_cur = valid_mask(A, s0, lane);
  commit(s0, ring0, wid, lane);
  commit_q(qst, sm.qs);
  __syncthreads();

  f32x4 O[8];
  float m_ref = -INFINITY, l_part = 0.0f;
  int64_t pend0 = -1, pend1 = -1;   // tokens whose partials this workgroup merges (<= 2)
  const float sl2 = A.scale_log2;
  const int head = kHeadGroup * hg + r16;

  auto step = [&](int i, Stage<kFp8>& freeS, Stage<kFp8>& nextS) {
    const int64_t c = c_lo + i;
    const int64_t t = c / cpt;
    const int cin = (int)(c - t * cpt);
    const bool seg_first = (i == 0) || (cin == 0);
    const bool seg_last = (i == n - 1) || (cin == cpt - 1);
    SMLA_LDS uint8_t* sb = (i & 1) ? ring1 : ring0;
    if (seg_first) {
#pragma unroll
      for (int k = 0; k < 8; k++) O[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_ref = -INFINITY;
      l_part = 0.0f;
    }
    // the next chunk starts a new token: fetch its query tile, committed after this chunk
    const bool next_new_tok = (i + 1 < n) && (cin == cpt - 1);
    if (next_new_tok) issue_q(A, t + 1, hg, qst);
    // prefetch chunk i+2 into the free register set, index list of chunk i+4
    if (i + 2 < n) {
      issue(A, c + 2, idx_a, freeS, wid, lane);
      idx_a = idx_b;
      idx_b = (i + 4 < n) ? load_idx(A, c + 4, wid, lane) : -1;
    }

    // ---- QK^T for rows 16*wid + r16 (A operand), 16 heads (B operand)
    const uint64_t vm = vm_cur;
    {
      const SMLA_LDS uint8_t* rp = sb + (kWaveRows * wid + r16) * F::kRB;
      // B operand of step k: query features 128g+8k.. (k < 16) or 512+16g+8(k-16)..
      auto qop = [&](int k) {
        return lds_load<f16x8>(&sm.qs[r16][k < 16 ? 128 * g + 8 * k : kLatent + 16 * g + 8 * (k - 16)]);
      };
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (!kFp8) {
        u32x4 cw[4];
#pragma unroll
        for (int k = 0; k < 4; k++) cw[k] = lds_load<u32x4>(rp + 64 * g + 16 * k);
        const u32x2 scb = lds_load<u32x2>(rp + kScaleOff + 8 * g);
        const u32x4 rb = lds_load<u32x4>(rp + kRopeOff + 16 * g);
        const f16x2 s01 = e4m3x2<false>(scb.x), s23 = e4m3x2<true>(scb.x);
        const f16x2 s45 = e4m3x2<false>(scb.y), s67 = e4m3x2<true>(scb.y);
        const f16 sf[8] = {s01.x, s01.y, s23.x, s23.y, s45.x, s45.y, s67.x, s67.y};
#pragma unroll
        for (int k = 0; k < 16; k++) {
          const f16 s = sf[k >> 1];
          acc = mfma16x16x32(unpack8(cw[k >> 2][k & 3], f16x2{s, s}), qop(k), acc);
          // keep the scheduler from hoisting every operand read ahead of the MFMA chain
          if ((k & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
        acc = mfma16x16x32(fp8x8(rb.x, rb.y), qop(16), acc);
        acc = mfma16x16x32(fp8x8(rb.z, rb.w), qop(17), acc);
        // scale table for PV: this wave's rows, empty rows scaled by zero
        const bool rv = (vm >> r16) & 1;
#pragma unroll
        for (int j = 0; j < 8; j++) sm.sc[8 * g + j][kWaveRows * wid + r16] = rv ? sf[j] : (f16)0.0f;
      } else {
        // FP8 row: latent bytes 128g.. (16 steps of 8), rope bytes 512+16g..
#pragma unroll
        for (int k = 0; k < 8; k++) {
          const u32x4 cw = lds_load<u32x4>(rp + 128 * g + 16 * k);
          acc = mfma16x16x32(fp8x8(cw.x, cw.y), qop(2 * k), acc);
          acc = mfma16x16x32(fp8x8(cw.z, cw.w), qop(2 * k + 1), acc);
        }
        const u32x4 rb = lds_load<u32x4>(rp + kLatent + 16 * g);
        acc = mfma16x16x32(fp8x8(rb.x, rb.y), qop(16), acc);
        acc = mfma16x16x32(fp8x8(rb.z, rb.w), qop(17), acc);
      }

      // acc[j] = score of row 16*wid + 4*g + j for head r16
      float sl[4];
#pragma unroll
      for (int j = 0; j < 4; j++) sl[j] = ((vm >> (4 * g + j)) & 1) ? acc[j] * sl2 : -INFINITY;
      float mx = fmaxf(fmaxf(sl[0], sl[1]), fmaxf(sl[2], sl[3]));
      mx = wave_max_xor16_32(mx);
      if (lane < kHeadGroup) sm.xmax[wid][lane] = mx;
      __syncthreads();
      const float cmax = fmaxf(fmaxf(sm.xmax[0][r16], sm.xmax[1][r16]),
                               fmaxf(sm.xmax[2][r16], sm.xmax[3][r16]));
      if (cmax > m_ref + kRescaleSlack) {
        const float alpha = exp2f(m_ref - cmax);   // 0 when m_ref = -inf
#pragma unroll
        for (int k = 0; k < 8; k++) O[k] *= alpha;
        l_part *= alpha;
        m_ref = cmax;
      }
      f16 p16[4];
      float psum = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float pv = (sl[j] == -INFINITY) ? 0.0f : exp2f(sl[j] - m_ref);
        p16[j] = (f16)pv;
        psum += (float)p16[j];
      }
      l_part += psum;
      lds_store<f16x4>(&sm.pb[r16][kWaveRows * wid + 4 * g], f16x4{p16[0], p16[1], p16[2], p16[3]});
    }
    __syncthreads();

    // ---- PV: O^T[16*tau + feature][head] += V^T P^T over the chunk's 64 rows
    {
      const f16x8 bop0 = lds_load<f16x8>(&sm.pb[r16][8 * g]);
      const f16x8 bop1 = lds_load<f16x8>(&sm.pb[r16][32 + 8 * g]);
      if constexpr (!kFp8) {
        // 4-bit transpose read: lane s of group g supplies row 8g+s (s < 8) or 32+8g+s-8;
        // dword 0 then holds rows 8g..8g+7 and dword 1 rows 32+8g.. of feature 16*tau+r16.
        const int trow = (r16 < 8) ? (8 * g + r16) : (32 + 8 * g + r16 - 8);
        const SMLA_LDS uint8_t* tp = sb + trow * kRowBytes;
#pragma unroll
        for (int k = 0; k < 8; k++) {
          const int tau = 8 * wid + k;
          const u32x2 d = lds_read_tr4(tp + 8 * tau);
          const f16x8 sc0 = lds_load<f16x8>(&sm.sc[tau][8 * g]);
          const f16x8 sc1 = lds_load<f16x8>(&sm.sc[tau][32 + 8 * g]);
          O[k] = mfma16x16x32(unpack8_pairs(d.x, sc0), bop0, O[k]);
          O[k] = mfma16x16x32(unpack8_pairs(d.y, sc1), bop1, O[k]);
        }
      } else {
        // 8-bit transpose read: lane s of group g supplies 8 bytes of row (8g + s/2) at
        // feature offset 8*(s%2); lane i receives feature 16*tau+i of rows 8g..8g+7.
        const SMLA_LDS uint8_t* tp0 = sb + (8 * g + (r16 >> 1)) * kHeadDim + 8 * (r16 & 1);
        const SMLA_LDS uint8_t* tp1 = tp0 + 32 * kHeadDim;
#pragma unroll
        for (int k = 0; k < 8; k++) {
          const int tau = 8 * wid + k;
          const u32x2 d0 = lds_read_tr8(tp0 + 16 * tau);
          const u32x2 d1 = lds_read_tr8(tp1 + 16 * tau);
          O[k] = mfma16x16x32(fp8x8(d0.x, d0.y), bop0, O[k]);
          O[k] = mfma16x16x32(fp8x8(d1.x, d1.y), bop1, O[k]);
        }
      }
    }

    // ---- stage the next chunk into the other LDS slot (its previous chunk is consumed)
    if (i + 1 < n) {
      vm_cur = valid_mask(A, nextS, lane);
      commit(nextS, (i & 1) ? ring0 : ring1, wid, lane);
    }
    if (next_new_tok) commit_q(qst, sm.qs);   // every wave is past its QK of this chunk

    // ---- epilogue of a token segment
    if (seg_last) {
      const float lw = wave_sum_xor16_32(l_part);
      if (lane < kHeadGroup) sm.lsum[wid][lane] = lw;
      __syncthreads();
      const float L = sm.lsum[0][r16] + sm.lsum[1][r16] + sm.lsum[2][r16] + sm.lsum[3][r16];
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      const float lse_nat = L > 0.0f ? (m_ref + log2f(L)) * kLn2 : -INFINITY;
      const int64_t tok0 = t * cpt;
      const bool full = (c_lo <= tok0) && (c_hi >= tok0 + cpt);
      if (full) {
        f16* op = (f16*)A.out + ((int64_t)t * A.H + head) * kLatent;
#pragma unroll
        for (int k = 0; k < 8; k++) {
          const f32x4 v = O[k] * inv;
          *(f16x4*)(op + 16 * (8 * wid + k) + 4 * g) = f16x4{(f16)v.x, (f16)v.y, (f16)v.z, (f16)v.w};
        }
        if (wid == 0 && lane < kHeadGroup) A.lse[(int64_t)t * A.H + head] = lse_nat;
      } else {
        const int64_t slot = ((int64_t)hg * G + w) * A.max_seg + (t - c_lo / cpt);
        float* po = A.part_o + (slot * kHeadGroup + r16) * kLatent;
#pragma unroll
        for (int k = 0; k < 8; k++) store_coherent(po + 16 * (8 * wid + k) + 4 * g, O[k] * inv);
        if (wid == 0 && lane < kHeadGroup) store_coherent(A.part_lse + slot * kHeadGroup + r16, lse_nat);
        // publish (stores complete), count, and let the last workgroup of this token merge
        const int64_t w_lo = wg_of_chunk(tok0, C, G), w_hi = wg_of_chunk(tok0 + cpt - 1, C, G);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
          int32_t* cnt = A.counters + (int64_t)hg * A.T + t;
          const int old = atomicAdd(cnt, 1);
          const int last = (old == (int)(w_hi - w_lo));
          if (last) atomicExch(cnt, 0);
          sm.flag = last;
        }
        __syncthreads();
        if (sm.flag) {   // merged after the main loop, outside the unrolled body
          if (pend0 < 0) pend0 = t; else pend1 = t;
        }
      }
    }
    __syncthreads();
  };

  for (int i = 0; i < n; i += 2) {
    step(i, s0, s1);
    if (i + 1 < n) step(i + 1, s1, s0);
  }

  // ---- log-sum-exp merge of the tokens this workgroup finished last
  for (int k = 0; k < 2; k++) {
    const int64_t t = k == 0 ? pend0 : pend1;
    if (t < 0) continue;
    const int64_t tok0 = t * cpt;
    const int64_t w_lo = wg_of_chunk(tok0, C, G), w_hi = wg_of_chunk(tok0 + cpt - 1, C, G);
    auto part = [&](int s, const float** o, const float** l) {
      const int64_t ws = w_lo + s;
      const int64_t sl = ((int64_t)hg * G + ws) * A.max_seg + (t - wg_first_chunk(ws, C, G) / cpt);
      *o = A.part_o + sl * kHeadGroup * kLatent;
      *l = A.part_lse + sl * kHeadGroup;
    };
    lse_merge16<true>((int)(w_hi - w_lo + 1), part,
                (f16*)A.out + ((int64_t)t * A.H + kHeadGroup * hg) * kLatent, kLatent,
                A.lse + (int64_t)t * A.H + kHeadGroup * hg);
  }
}

__global__ __launch_bounds__(256) void sparse_mla_combine_kernel(const float* __restrict__ part_o,
                                                                 const float* __restrict__ part_lse,
                                                                 int32_t T, int32_t S, int32_t H,
                                                                 f16* __restrict__ out,
                                                                 float* __restrict__ lse) {
  const int t = blockIdx.x, hg = blockIdx.y;
  auto part = [&](int s, const float** o, const float** l) {
    const int64_t base = ((int64_t)t * S + s) * H + kHeadGroup * hg;
    *o = part_o + base * kLatent;
    *l = part_lse + base;
  };
  lse_merge16<false>(S, part, out + ((int64_t)t * H + kHeadGroup * hg) * kLatent, kLatent,
              lse + (int64_t)t * H + kHeadGroup * hg);
}

hipError_t launch_decode_nvfp4(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(sparse_mla_decode_kernel<false>, dim3(a.G, a.H / kHeadGroup), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_fp8rows(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(sparse_mla_decode_kernel<true>, dim3(a.G, a.H / kHeadGroup), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const float* part_o, const float* part_lse, int32_t T, int32_t S,
                          int32_t H, void* out, float* lse, hipStream_t s) {
  hipLaunchKernelGGL(sparse_mla_combine_kernel, dim3(T, H / kHeadGroup), dim3(256), 0, s, part_o,
                     part_lse, T, S, H, (f16*)out, lse);
  return hipGetLastError();
}

}  // namespace smla

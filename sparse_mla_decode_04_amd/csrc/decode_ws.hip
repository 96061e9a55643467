// Fused sparse MLA decode over NVFP4 cache rows with waves specialised by role: scoring
// waves and accumulating waves (gfx950 / MI355X).  One kernel template for head blocks of
// 64 (the default at 64 and more heads) and of 16.
//
// "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section
// "Four-bit caches make room": per decode token, only the cache rows named by the sparse
// indexer's list are loaded, the NVFP4 values are unpacked on chip, attention runs with
// FP16 operands and FP32 accumulation, and empty list entries are handled.  The page's
// kernel overlaps unpacking with scoring and accumulation by giving the stages to
// different warp groups; this kernel does the same with two roles of four waves each.
//
// One workgroup of eight waves per CU; each SIMD runs one scoring wave and one
// accumulating wave, which issue into its VALU and matrix core in turn.
//
//  * Step s (one barrier per step): the scoring waves score tile s while the accumulating
//    waves apply the probabilities of tile s-1 to its rows.
//  * Gather (scoring waves): the rows of tile s+2 are fetched by LDS DMA into a ring of
//    four slots (tile s-1 being accumulated, tile s being scored, two in flight); scoring
//    wave w fetches rows 16w..16w+15 of a tile, piece-major; empty entries read as zeros
//    without a memory access; index entries run two tiles ahead of the rows.
//  * QK^T: the scoring waves cover the tile's 64 rows x NH heads as RG row groups x HW head
//    groups; scoring wave w takes row group w % RG (MT tiles of 16 rows) and head group
//    w / RG (JT tiles of 16 heads).  NH = 64: 32 rows x 32 heads per wave (each row
//    unpacked by two waves) as one v_mfma_f32_32x32x16_f16 tile, each 16-byte ring read
//    feeding four MFMAs; NH = 16: 16 rows x 16 heads on v_mfma_f32_16x16x32_f16.
//  * Softmax per head over the tile's 64 rows, shared between the row groups through a
//    per-head reference in LDS (a row group keeps the shared reference unless its rows
//    exceed it by more than the slack); probabilities and the rows' group scales to LDS.
//  * PV (accumulating wave p): output features 128p..128p+127 for all NH heads,
//    O^T += V^T P^T; each unpacked V^T fragment (4-bit transpose read of the ring, times
//    the group scales) feeds NH/16 pairs of MFMAs.
//  * Split epilogue as in the other kernels; the in-launch merge runs as two teams of four
//    waves (NH = 64: 32 heads each; NH = 16: the first team, the second joins its barriers).
//
// With kFp8 (NH = 64) the kernel attends over 576-byte FP8 E4M3 rows instead: the rows
// pass 1 of the staged variant wrote to HBM (one per list entry) or the rows of a pool kept
// in FP8.  E4M3 -> fp16 is exact and takes one conversion per pair of values, with no group
// scales; PV reads V^T through the 8-bit LDS transpose read.  The 512-byte latent goes to
// the four-slot ring and the 64-byte rope to a three-slot ring of its own: only QK^T reads
// the rope, in the step that scores the tile, and a four-slot ring of whole rows would not
// leave room in LDS for the probability tables.
#include "smla_launch.hpp"
#include "smla_tile.hpp"

namespace smla {

namespace {

constexpr int kST = 4;                    // ring slots
constexpr int kThreads = 2 * kWaves * 64; // scoring waves 0..3, accumulating waves 4..7

// Ring layout of a row format.  NVFP4: the whole 352-byte row in the ring (pieces 0..15
// codes, 16..17 scales, 18..21 rope).  FP8: the latent (pieces 0..31) in the ring, the rope
// in the rope ring.
template <bool kFp8>
struct WsFmt {
  static constexpr int kPieces = kFp8 ? kLatent / 16 : kRowBytes / 16;   // 32 or 22
  static constexpr int kLoads = (kPieces + 3) / 4;     // ring DMA per scoring wave per tile: 8 or 6
  static constexpr int kPortion = kPieces * 256;       // one scoring wave's 16 rows, [piece][row]
  static constexpr int kSlot = kWaves * kPortion;      // one tile
  static constexpr int kRopeST = kFp8 ? 3 : 0;         // rope ring slots
  static constexpr int kRopePortion = 4 * 256;         // 16 rows x 4 pieces of rope
  static constexpr int kRopeSlot = kWaves * kRopePortion;
  static constexpr int kVmOps = kLoads + (kFp8 ? 1 : 0);   // vector memory instructions per tile
  static constexpr int kRingBytes = kST * kSlot + kRopeST * kRopeSlot;
};

template <int NH>
struct WsShape {
  static_assert(NH == 16 || NH == 64, "head block");
  static constexpr int JT = NH == 64 ? 2 : 1;   // 16-head tiles per scoring wave
  static constexpr int HW = NH / (16 * JT);     // head groups of scoring waves
  static constexpr int RG = kWaves / HW;        // row groups of scoring waves
  static constexpr int MT = 4 / RG;             // 16-row tiles per scoring wave
  static constexpr int NJ = NH / 16;            // 16-head tiles of an accumulating wave
};

template <int NH, bool kGrouped, bool kFp8>
struct __attribute__((aligned(16))) SmemWs {
  // [slot][portion][piece][row] 16-byte pieces, then (FP8) the rope ring [slot][portion][piece][row]
  uint8_t ring[WsFmt<kFp8>::kRingBytes];
  uint8_t members[(kGrouped || !kFp8) ? kST : 1][kTileRows];   // grouped decode: member bits [slot][row]
  int32_t idx[2][kWaves][kWR];            // index-list DMA landing zone [tile parity][portion]
  f16 sc[2][kFp8 ? 1 : 32][kPH];          // NVFP4 PV scales [parity][group][tile row]
  f16 pb[2][NH][kPH];                     // probabilities [parity][head][tile row]
  float wref[2][WsShape<NH>::RG][NH];     // reference each row group used [parity][group][head]
  int wflag[2][kWaves];                   // bit 0: wave raised a reference; bit 1: wave has a row
  uint32_t vmask[kST][kWaves];            // valid rows of each DMA portion [slot][portion]
  int flag;
};

// The lane id behind an empty volatile asm: per-lane addresses derived from it inside the
// tile loop are recomputed each tile instead of being hoisted into registers that stay live
// across the whole loop (the query and the accumulators leave little room).
__device__ __forceinline__ int fresh_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

}  // namespace

// kGrouped: the index entries are union-list entries of token groups (row | members << 27),
// the NH = 64 heads are those of the group's tokens (A.tok_heads heads each), and a score
// counts only where the head's token lists the row.
template <int NH, bool kGrouped, bool kFp8>
__global__ __launch_bounds__(kThreads, 1) void sparse_mla_decode_ws_kernel(DecodeArgs A) {
  using S = WsShape<NH>;
  using F = WsFmt<kFp8>;
  constexpr int JT = S::JT, RG = S::RG, MT = S::MT, NJ = S::NJ;
  // 64-head blocks score with 32x32x16 MFMAs (a scoring wave's 32 rows x 32 heads are one
  // tile); 16-head blocks with 16x16x32
  constexpr bool kM32 = NH == 64;
  static_assert(!kFp8 || (NH == 64 && !kGrouped), "FP8 rows: 64-head blocks, per-token lists");
  static_assert(sizeof(SmemWs<NH, kGrouped, kFp8>) <= 160 * 1024, "LDS of one CU");
  __shared__ SmemWs<NH, kGrouped, kFp8> sm;
  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // XCD-aware order (see the other kernels).
  const int nb = gridDim.x, b = blockIdx.x, xcd = b & 7, per = nb >> 3, rem = nb & 7;
  const int L = xcd * per + min(xcd, rem) + (b >> 3);
  const int w = L / A.HB, hb = L - w * A.HB;
  const int64_t C = A.tiles;
  const int G = A.G;
  const int cpt = A.cpt;
  const int64_t c_lo = wg_first_chunk(w, C, G), c_hi = wg_first_chunk(w + 1, C, G);
  const int n = (int)(c_hi - c_lo);
  const int head0 = hb * NH;
  SMLA_LDS uint8_t* const ring = (SMLA_LDS uint8_t*)sm.ring;
  SMLA_LDS uint8_t* const rope_ring = ring + kST * F::kSlot;   // FP8 only
  const __amdgpu_buffer_rsrc_t ws_o = merge_rsrc(A.part_o, A.part_o_bytes);
  const __amdgpu_buffer_rsrc_t ws_l = merge_rsrc(A.part_lse, A.part_lse_bytes);

  if (wid < kWaves) {
    // =============================== scoring waves ===============================
    const int rg = wid % RG, hg = wid / RG;   // row group, head group
    const float sl2 = A.scale_log2;
    const i32x4 rs_rows = make_rsrc(A.rows, A.rows_bytes);
    const i32x4 rs_idx = make_rsrc(A.idx, A.idx_bytes);
    SMLA_LDS int32_t* const idxbuf = (SMLA_LDS int32_t*)sm.idx;

    // DMA of this wave's 16 index entries of tile cur (relative index i) into idx[i & 1][wid].
    auto issue_idx = [&](const Cursor& cur, int i, int ln) {
      const int k = cur.ci * kTileRows + kWR * wid + ln;
      const bool ok = cur.c < c_hi && k < A.topk;
      const uint32_t voff = ok ? (uint32_t)(cur.t * A.topk + k) * 4u : kOOB;
      if (ln < kWR) dma4(rs_idx, voff, lds_addr(idxbuf + ((i & 1) * kWaves + wid) * kWR));
    };
    // Index entry of this wave's row r16 of tile i (its DMA must have landed).
    auto idx_entry = [&](int i, int ln) { return idxbuf[((i & 1) * kWaves + wid) * kWR + (ln & 15)]; };
    // DMA of this wave's rows of tile cur into ring slot i % 4 (FP8: and their rope into
    // rope slot i % 3), e = the lane's index entry.  Issued in step i-2: the slot last held
    // tile i-4, accumulated in step i-3, before the barrier that ended it (the rope slot:
    // tile i-3, scored in step i-3).  prep_rows takes the lane's row address and writes the
    // portion's valid-row mask to sm.vmask (and, grouped, the member bits);
    // row_dma(rd, d) issues DMA instruction d of the F::kVmOps (ring pieces 4d .. 4d+3; FP8
    // d = F::kLoads: the rope).
    struct RowDma {
      uint32_t base;   // byte offset of the lane's row (unused where !ok)
      bool ok;
      int slot;        // tile i
    };
    auto prep_rows = [&](const Cursor& cur, int i, int ln, int32_t e) -> RowDma {
      const int r16 = ln & 15, g = ln >> 4;
      const int k = cur.ci * kTileRows + kWR * wid + r16;
      const int32_t v = kGrouped ? (e < 0 ? -1 : (e & kRowMask)) : e;
      const bool ok = cur.c < c_hi && k < A.topk && row_valid(v, A.pool_rows);
      if (kGrouped && g == 0) sm.members[i % kST][kWR * wid + r16] = ok ? (uint8_t)(e >> kMemberShift) : 0;
      // FP8: row v of a pool, or the staged row of entry (t, k)
      const uint32_t base = kFp8 ? (uint32_t)(A.fp8_pool ? (int64_t)v : cur.t * A.topk + k) * (uint32_t)kHeadDim
                                 : storage_row((uint32_t)v, A.map) * (uint32_t)kRowBytes;
      const uint32_t vm = (uint32_t)__ballot(ok && g == 0) & 0xFFFFu;
      if (ln == 0) sm.vmask[i % kST][wid] = vm;
      return RowDma{base, ok, i};
    };
    auto row_dma = [&](const RowDma& rd, int d, int ln) {
      const int g = ln >> 4;
      if (d < F::kLoads) {
        const int piece = 4 * d + g;
        const uint32_t voff = rd.ok ? rd.base + 16u * piece : kOOB;
        const uint32_t lds0 = lds_addr(ring + (rd.slot % kST) * F::kSlot + wid * F::kPortion);
        if (4 * d + 3 < F::kPieces || piece < F::kPieces) dma16(rs_rows, voff, lds0 + 1024u * d);
      } else if (kFp8 && d == F::kLoads) {
        const uint32_t voff = rd.ok ? rd.base + (uint32_t)kLatent + 16u * g : kOOB;
        dma16(rs_rows, voff, lds_addr(rope_ring + (rd.slot % F::kRopeST) * F::kRopeSlot + wid * F::kRopePortion));
      }
    };
    auto issue_rows = [&](const Cursor& cur, int i, int ln, int32_t e) {
      const RowDma rd = prep_rows(cur, i, ln, e);
#pragma unroll
      for (int d = 0; d < F::kVmOps; d++) row_dma(rd, d, ln);
    };

    // Query registers of the wave's 16*JT heads.  16x16x32: Q[j][k] = B operand of QK step
    // k for head 16*JT*hg + 16j + r16 (latent features 128g + 8k.., rope 512 + 16g +
    // 8(k-16)..).  32x32x16: chunk c = Qc(c) is the B operand for head 32hg + (ln & 31), K
    // half kh = ln >> 5: latent features 256kh + 8c .. +7 (c < 32), rope 512 + 32kh +
    // 8(c - 32) .. +7 (c = 32 .. 35).
    f16x8 Q[JT][18];
    auto Qc = [&](int c) -> f16x8& { return Q[c / 18][c % 18]; };
    auto load_q = [&](int64_t t, int ln) {
      if constexpr (kM32) {
        const int kh = ln >> 5;
        const f16* base = (const f16*)A.q + ((t * A.H + head0 + 32 * hg + (ln & 31)) * kHeadDim);
#pragma unroll
        for (int c = 0; c < 32; c++) Qc(c) = *(const f16x8*)(base + 256 * kh + 8 * c);
#pragma unroll
        for (int c = 0; c < 4; c++) Qc(32 + c) = *(const f16x8*)(base + kLatent + 32 * kh + 8 * c);
      } else {
        const int r16 = ln & 15, g = ln >> 4;
#pragma unroll
        for (int j = 0; j < JT; j++) {
          const f16* base = (const f16*)A.q + ((t * A.H + head0 + 16 * JT * hg + 16 * j + r16) * kHeadDim);
#pragma unroll
          for (int k = 0; k < 16; k++) Q[j][k] = *(const f16x8*)(base + 128 * g + 8 * k);
          Q[j][16] = *(const f16x8*)(base + kLatent + 16 * g);
          Q[j][17] = *(const f16x8*)(base + kLatent + 16 * g + 8);
        }
      }
    };

    // ---- prologue: query, index entries of tiles 0 and 1, rows of tiles 0 and 1 with
    // index entries of tiles 2 and 3.  Order of this wave's vector memory operations from
    // here on: ..., rows(i), idx(i+2), rows(i+1), idx(i+3), ...
    Cursor cr, cx, cu;   // next row DMA (tile s+2), next index DMA (tile s+4), tile s
    cr.init(c_lo, cpt);
    cx.init(c_lo, cpt);
    cu.init(c_lo, cpt);
    load_q(cu.t, lane);
    issue_idx(cx, 0, lane);
    cx.next(cpt);
    issue_idx(cx, 1, lane);
    cx.next(cpt);
    wait_vm<0>();
#pragma unroll
    for (int d = 0; d < 2; d++) {
      issue_rows(cr, d, lane, idx_entry(d, lane));
      cr.next(cpt);
      issue_idx(cx, d + 2, lane);
      cx.next(cpt);
    }
    wait_vm<F::kVmOps + 1>();   // rows(0), idx(2) have landed
    __syncthreads();         // every portion of tile 0 has landed

    float mq[JT];   // shared reference of head 16*JT*hg + 16j + r16 (32x32x16: mq[0], the lane's head)
#pragma unroll
    for (int j = 0; j < JT; j++) mq[j] = -INFINITY;
    for (int s = 0; s <= n; s++) {
      if (s < n) {
        const int par = s & 1;
        const SMLA_LDS uint8_t* const slot = ring + (s % kST) * F::kSlot;
        const int ln = fresh_lane(lane), r16 = ln & 15, g = ln >> 4;
        const bool new_seg = cu.ci == 0;
        if (new_seg) {
          // the first tile of a token starts a new segment; a later token's query is
          // loaded here (with it every DMA issued so far completes)
#pragma unroll
          for (int j = 0; j < JT; j++) mq[j] = -INFINITY;
          if (s > 0) {
            load_q(cu.t, ln);
            wait_vm<0>();
          }
        }

        // LDS reads the step needs after QK^T, issued first so that QK^T covers their latency:
        // the index entry of tile s+2 (landed by the last barrier; its slot is refilled by
        // the DMA for tile s+4 issued later in this step) and the flags of tile s-1
        const int32_t e_next = idx_entry(s + 2, ln);
        const int pp = par ^ 1;
        const int fl_prev = sm.wflag[pp][0] | sm.wflag[pp][1] | sm.wflag[pp][2] | sm.wflag[pp][3];
        // This step's gather (rows of tile s+2, then index entries of tile s+4): the
        // F::kVmOps + 1 DMA instructions are spread over QK^T, so that the CU's address
        // unit takes them while the matrix work runs instead of in one burst per wave.
        const RowDma rd = prep_rows(cr, s + 2, ln, e_next);
        auto gather = [&](int d) {
          if (d < F::kVmOps) row_dma(rd, d, ln);
          else if (d == F::kVmOps) issue_idx(cx, s + 4, ln);
        };

        // ---- QK^T: rows 16*MT*rg + 16m + r16 against heads 16*JT*hg + 16j + r16
        uint32_t vrow = 0;   // bit 16m + r: row 16*MT*rg + 16m + r is valid
#pragma unroll
        for (int m = 0; m < MT; m++) vrow |= sm.vmask[s % kST][MT * rg + m] << (16 * m);
        bool raised = false;
        if constexpr (kM32) {
          // 32x32x16 MFMAs.  Lane (row 32rg + (ln & 31), K half kh = ln >> 5) supplies the A
          // operand of chunk c: eight latent values 256kh + 8c .. +7 of one scale group (c <
          // 32), or rope values 32kh + 8(c - 32) .. +7 (c = 32 .. 35).  Accumulator element i
          // is the score of row 8(i/4) + 4kh + i%4 of the wave's 32 against head 32hg + (ln & 31).
          const int row = ln & 31, kh = ln >> 5;
          const int hl = 32 * hg + row;   // the lane's head in the block
          uint32_t mrow4[4];              // grouped: member bytes of rows 8b + 4kh .. +3
          if constexpr (kGrouped) {
#pragma unroll
            for (int b = 0; b < 4; b++)
              mrow4[b] = lds_load<uint32_t>(&sm.members[s % kST][32 * rg + 8 * b + 4 * kh]);
          }
          f32x16 acc = f32x16{};
          f16x2 sp[8];   // NVFP4 group scales of the lane's row: sp[i] = groups 16kh + 2i, +1
          const SMLA_LDS uint8_t* const por = slot + (2 * rg + (row >> 4)) * F::kPortion + 16 * (row & 15);
          if (kFp8 && vrow != 0) {
            // FP8: chunk c of half kh is bytes 256kh + 8c .. +7, piece 16kh + c/2
#pragma unroll
            for (int pc = 0; pc < 16; pc++) {
              gather(pc);
              const u32x4 cw = lds_load<u32x4>(por + 256 * (16 * kh + pc));
              acc = mfma32x32x16(fp8x8(cw.x, cw.y), Qc(2 * pc), acc);
              acc = mfma32x32x16(fp8x8(cw.z, cw.w), Qc(2 * pc + 1), acc);
            }
            const SMLA_LDS uint8_t* const rpor = rope_ring + (s % F::kRopeST) * F::kRopeSlot +
                                                 (2 * rg + (row >> 4)) * F::kRopePortion + 16 * (row & 15);
            const u32x4 r0 = lds_load<u32x4>(rpor + 256 * (2 * kh)), r1 = lds_load<u32x4>(rpor + 256 * (2 * kh + 1));
            acc = mfma32x32x16(fp8x8(r0.x, r0.y), Qc(32), acc);
            acc = mfma32x32x16(fp8x8(r0.z, r0.w), Qc(33), acc);
            acc = mfma32x32x16(fp8x8(r1.x, r1.y), Qc(34), acc);
            acc = mfma32x32x16(fp8x8(r1.z, r1.w), Qc(35), acc);
          } else if (!kFp8 && vrow != 0) {
            // NVFP4: the half row's 16 group scales are scale bytes 16kh .. 16kh+15 (piece
            // 16 + kh); its codes are pieces 8kh .. 8kh+7 (four chunks each); its rope is
            // pieces 18 + 2kh and 19 + 2kh
            const u32x4 scb = lds_load<u32x4>(por + 256 * (16 + kh));
            sp[0] = e4m3x2<false>(scb.x);
            sp[1] = e4m3x2<true>(scb.x);
            sp[2] = e4m3x2<false>(scb.y);
            sp[3] = e4m3x2<true>(scb.y);
            sp[4] = e4m3x2<false>(scb.z);
            sp[5] = e4m3x2<true>(scb.z);
            sp[6] = e4m3x2<false>(scb.w);
            sp[7] = e4m3x2<true>(scb.w);
#pragma unroll
            for (int q = 0; q < 8; q++) {
              gather(q);
              const u32x4 cw = lds_load<u32x4>(por + 256 * (8 * kh + q));
#pragma unroll
              for (int kk = 0; kk < 4; kk++) {
                const int c = 4 * q + kk;   // group 16kh + c/2
                const f16 sk = ((c >> 1) & 1) ? sp[c >> 2].y : sp[c >> 2].x;
                acc = mfma32x32x16(unpack8(cw[kk], f16x2{sk, sk}), Qc(c), acc);
              }
            }
            const u32x4 r0 = lds_load<u32x4>(por + 256 * (18 + 2 * kh)), r1 = lds_load<u32x4>(por + 256 * (19 + 2 * kh));
            acc = mfma32x32x16(fp8x8(r0.x, r0.y), Qc(32), acc);
            acc = mfma32x32x16(fp8x8(r0.z, r0.w), Qc(33), acc);
            acc = mfma32x32x16(fp8x8(r1.x, r1.y), Qc(34), acc);
            acc = mfma32x32x16(fp8x8(r1.z, r1.w), Qc(35), acc);
          } else {
#pragma unroll
            for (int d = 0; d <= F::kVmOps; d++) gather(d);
#pragma unroll
            for (int i = 0; i < 8; i++) sp[i] = f16x2{(f16)0.0f, (f16)0.0f};
          }
          // PV scale table: both waves of a row group hold its rows' scales; head group hg
          // writes groups 16kh + 8hg .. +7 (an empty row was fetched as zeros, so its scales
          // are 0), picking its half of the registers by a select, not a branch.
          if constexpr (!kFp8) {
#pragma unroll
            for (int jj = 0; jj < 8; jj++) {
              const f16x2 v = hg ? sp[4 + (jj >> 1)] : sp[jj >> 1];
              sm.sc[par][16 * kh + 8 * hg + jj][32 * rg + row] = (jj & 1) ? v.y : v.x;
            }
          }

          cr.next(cpt);
          cx.next(cpt);

          // ---- shared reference of the lane's head after tile s-1 of the same segment: the
          // largest one the row groups used
          if (s > 0 && !new_seg && (fl_prev & 1)) {
            float m = sm.wref[pp][0][hl];
#pragma unroll
            for (int q = 1; q < RG; q++) m = fmaxf(m, sm.wref[pp][q][hl]);
            mq[0] = m;
          }

          // ---- softmax over the lane's 16 rows and its partner lane's (ln ^ 32) 16, as below
          const bool all_valid = !kGrouped && vrow == 0xFFFFFFFFu;
          const int tok = kGrouped ? hl / A.tok_heads : 0;
          float sv[16];
#pragma unroll
          for (int i = 0; i < 16; i++) {
            if (all_valid) {
              sv[i] = acc[i];
            } else {
              bool valid = (vrow >> (8 * (i >> 2) + 4 * kh + (i & 3))) & 1;
              if constexpr (kGrouped) valid = valid && ((mrow4[i >> 2] >> (8 * (i & 3) + tok)) & 1);
              sv[i] = valid ? acc[i] : -INFINITY;
            }
          }
          float mx = sv[0];
#pragma unroll
          for (int i = 1; i < 16; i++) mx = fmaxf(mx, sv[i]);
          mx = wave_max_xor32(mx * sl2);   // scale_log2 > 0: the scaled maximum
          const float ref = (mx > mq[0] + kSlack) ? mx : mq[0];
          raised = ref != mq[0];
          const float nref = (ref == -INFINITY) ? 0.0f : -ref;
#pragma unroll
          for (int b = 0; b < 4; b++) {
            f16 pr[4];
#pragma unroll
            for (int ii = 0; ii < 4; ii++) pr[ii] = (f16)__builtin_amdgcn_exp2f(fmaf(sv[4 * b + ii], sl2, nref));
            lds_store<f16x4>(&sm.pb[par][hl][32 * rg + 8 * b + 4 * kh], f16x4{pr[0], pr[1], pr[2], pr[3]});
          }
          sm.wref[par][rg][hl] = ref;
        } else {
          // grouped: byte jj of mrow[m] holds the member bits of row 16*MT*rg + 16m + 4g + jj
          uint32_t mrow[MT];
          if constexpr (kGrouped) {
#pragma unroll
            for (int m = 0; m < MT; m++)
              mrow[m] = lds_load<uint32_t>(&sm.members[s % kST][16 * MT * rg + 16 * m + 4 * g]);
          }
          f32x4 acc[MT][JT];
#pragma unroll
          for (int m = 0; m < MT; m++)
#pragma unroll
            for (int j = 0; j < JT; j++) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
          f16x2 sp[MT][4];   // group scales of the lane's rows: sp[m][q] = groups 8g+2q, 8g+2q+1
          if (kFp8 && vrow != 0) {
            // FP8: K step k reads latent features 128g + 8k .. +7 of the row: 16-byte piece
            // 8g + k/2, half k%2
#pragma unroll
            for (int kp = 0; kp < 8; kp++) {
              gather(kp);
              u32x4 cw[MT];
#pragma unroll
              for (int m = 0; m < MT; m++)
                cw[m] = lds_load<u32x4>(slot + (MT * rg + m) * F::kPortion + 256 * (8 * g + kp) + 16 * r16);
#pragma unroll
              for (int kk = 0; kk < 2; kk++) {
#pragma unroll
                for (int m = 0; m < MT; m++) {
                  const f16x8 a = fp8x8(cw[m][2 * kk], cw[m][2 * kk + 1]);
#pragma unroll
                  for (int j = 0; j < JT; j++) acc[m][j] = mfma16x16x32(a, Q[j][2 * kp + kk], acc[m][j]);
                }
              }
            }
            gather(8);
            gather(9);
            const SMLA_LDS uint8_t* const rslot = rope_ring + (s % F::kRopeST) * F::kRopeSlot;
#pragma unroll
            for (int m = 0; m < MT; m++) {
              const u32x4 rb = lds_load<u32x4>(rslot + (MT * rg + m) * F::kRopePortion + 256 * g + 16 * r16);
              const f16x8 r0 = fp8x8(rb.x, rb.y), r1 = fp8x8(rb.z, rb.w);
#pragma unroll
              for (int j = 0; j < JT; j++) {
                acc[m][j] = mfma16x16x32(r0, Q[j][16], acc[m][j]);
                acc[m][j] = mfma16x16x32(r1, Q[j][17], acc[m][j]);
              }
            }
          } else if (!kFp8 && vrow != 0) {
#pragma unroll
            for (int m = 0; m < MT; m++) {
              const SMLA_LDS uint8_t* por = slot + (MT * rg + m) * F::kPortion + 16 * r16;
              const u32x2 scb = lds_load<u32x2>(por + 256 * (16 + (g >> 1)) + 8 * (g & 1));
              sp[m][0] = e4m3x2<false>(scb.x);
              sp[m][1] = e4m3x2<true>(scb.x);
              sp[m][2] = e4m3x2<false>(scb.y);
              sp[m][3] = e4m3x2<true>(scb.y);
            }
#pragma unroll
            for (int kq = 0; kq < 4; kq++) {
              gather(2 * kq);
              gather(2 * kq + 1);
              u32x4 cw[MT];
#pragma unroll
              for (int m = 0; m < MT; m++)
                cw[m] = lds_load<u32x4>(slot + (MT * rg + m) * F::kPortion + 256 * (4 * g + kq) + 16 * r16);
#pragma unroll
              for (int kk = 0; kk < 4; kk++) {
                const int k = 4 * kq + kk;
#pragma unroll
                for (int m = 0; m < MT; m++) {
                  const f16 sk = (k & 2) ? sp[m][k >> 2].y : sp[m][k >> 2].x;
                  const f16x8 a = unpack8(cw[m][kk], f16x2{sk, sk});
#pragma unroll
                  for (int j = 0; j < JT; j++) acc[m][j] = mfma16x16x32(a, Q[j][k], acc[m][j]);
                }
              }
            }
#pragma unroll
            for (int m = 0; m < MT; m++) {
              const u32x4 rb = lds_load<u32x4>(slot + (MT * rg + m) * F::kPortion + 256 * (18 + g) + 16 * r16);
              const f16x8 r0 = fp8x8(rb.x, rb.y), r1 = fp8x8(rb.z, rb.w);
#pragma unroll
              for (int j = 0; j < JT; j++) {
                acc[m][j] = mfma16x16x32(r0, Q[j][16], acc[m][j]);
                acc[m][j] = mfma16x16x32(r1, Q[j][17], acc[m][j]);
              }
            }
          } else {
#pragma unroll
            for (int d = 0; d <= F::kVmOps; d++) gather(d);
#pragma unroll
            for (int m = 0; m < MT; m++)
#pragma unroll
              for (int q = 0; q < 4; q++) sp[m][q] = f16x2{(f16)0.0f, (f16)0.0f};
          }
          // PV scale table: the head-group-0 waves write their rows' scales (an empty row was
          // fetched as zeros, so its scales are 0)
          if (!kFp8 && hg == 0) {
#pragma unroll
            for (int m = 0; m < MT; m++) {
              const int row = 16 * MT * rg + 16 * m + r16;
#pragma unroll
              for (int jj = 0; jj < 8; jj++)
                sm.sc[par][8 * g + jj][row] = (jj & 1) ? sp[m][jj >> 1].y : sp[m][jj >> 1].x;
            }
          }

          cr.next(cpt);
          cx.next(cpt);

          // ---- shared references after tile s-1 of the same segment: the largest one the
          // row groups used
          if (s > 0 && !new_seg) {
            if (fl_prev & 1) {
#pragma unroll
              for (int j = 0; j < JT; j++) {
                const int h = 16 * JT * hg + 16 * j + r16;
                float m = sm.wref[pp][0][h];
#pragma unroll
                for (int q = 1; q < RG; q++) m = fmaxf(m, sm.wref[pp][q][h]);
                mq[j] = m;
              }
            }
          }

          // ---- softmax.  acc[m][j][jj] = score of row 16*MT*rg + 16m + 4g + jj, head
          // 16*JT*hg + 16j + r16.
          // Scores enter as exp2(score * scale_log2 - ref) in one fma each; an invalid row
          // enters as -inf (exp2 gives 0), and a head with no valid row takes 0 for -ref.
          // When every row of the wave is valid (and no member bits apply) no mask is needed.
          const bool all_valid = !kGrouped && vrow == (MT == 2 ? 0xFFFFFFFFu : 0xFFFFu);
#pragma unroll
          for (int j = 0; j < JT; j++) {
            float sv[MT][4];
            // grouped: the token (within the group) of heads 16*JT*hg + 16j ..
            const int tok = kGrouped ? (16 * JT * hg + 16 * j) / A.tok_heads : 0;
#pragma unroll
            for (int m = 0; m < MT; m++)
#pragma unroll
              for (int jj = 0; jj < 4; jj++) {
                if (all_valid) {
                  sv[m][jj] = acc[m][j][jj];
                } else {
                  bool valid = (vrow >> (16 * m + 4 * g + jj)) & 1;
                  if constexpr (kGrouped) valid = valid && ((mrow[m] >> (8 * jj + tok)) & 1);
                  sv[m][jj] = valid ? acc[m][j][jj] : -INFINITY;
                }
              }
            float mx = sv[0][0];
#pragma unroll
            for (int m = 0; m < MT; m++)
#pragma unroll
              for (int jj = 0; jj < 4; jj++) mx = fmaxf(mx, sv[m][jj]);
            mx = wave_max_xor16_32(mx * sl2);   // scale_log2 > 0: the scaled maximum
            const float ref = (mx > mq[j] + kSlack) ? mx : mq[j];
            raised |= ref != mq[j];
            const float nref = (ref == -INFINITY) ? 0.0f : -ref;
            const int h = 16 * JT * hg + 16 * j + r16;
#pragma unroll
            for (int m = 0; m < MT; m++) {
              f16 p[4];
#pragma unroll
              for (int jj = 0; jj < 4; jj++) p[jj] = (f16)__builtin_amdgcn_exp2f(fmaf(sv[m][jj], sl2, nref));
              lds_store<f16x4>(&sm.pb[par][h][16 * MT * rg + 16 * m + 4 * g], f16x4{p[0], p[1], p[2], p[3]});
            }
            sm.wref[par][rg][h] = ref;
          }
        }
        const bool wave_raised = __ballot(raised) != 0;
        sm.wflag[par][wid] = (wave_raised ? 1 : 0) | (vrow != 0 ? 2 : 0);
        cu.next(cpt);
        wait_vm<F::kVmOps + 1>();   // rows(s+1), idx(s+3) have landed
      }
      __syncthreads();
    }
  } else {
    // ============================= accumulating waves =============================
    const int pw = wid - kWaves;   // output features 128pw .. 128pw + 127
    // O[tau][j4]: O^T for features 128pw + 16tau + 4g .. +3 of head 16*j4 + r16.
    // m_ref[j4], l_acc[j4]: reference and the lane's share of the denominator of that head.
    f32x4 O[8][NJ];
    float m_ref[NJ], l_acc[NJ];
#pragma unroll
    for (int j4 = 0; j4 < NJ; j4++) {
#pragma unroll
      for (int k = 0; k < 8; k++) O[k][j4] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_ref[j4] = -INFINITY;
      l_acc[j4] = 0.0f;
    }
    Cursor cu;   // tile s-1
    cu.init(c_lo, cpt);
    const int64_t t_first = cu.t;
    __syncthreads();   // the scoring waves' prologue

    for (int s = 0; s <= n; s++) {
      if (s > 0) {
        const int par = (s - 1) & 1;
        const SMLA_LDS uint8_t* const slot = ring + ((s - 1) % kST) * F::kSlot;
        const int ln = fresh_lane(lane), r16 = ln & 15, g = ln >> 4;
        // ---- PV operand: probabilities of all NH heads, rows 8g..8g+7 (half 0) and
        // 32+8g.. (half 1); those rows belong to row group rgh[half]
        const int fl = sm.wflag[par][0] | sm.wflag[par][1] | sm.wflag[par][2] | sm.wflag[par][3];
        f16x8 bop[NJ][2];
#pragma unroll
        for (int j4 = 0; j4 < NJ; j4++) {
          bop[j4][0] = lds_load<f16x8>(&sm.pb[par][16 * j4 + r16][8 * g]);
          bop[j4][1] = lds_load<f16x8>(&sm.pb[par][16 * j4 + r16][32 + 8 * g]);
        }
        if (fl & 1) {
          // a row group raised its reference: the new shared reference of a head is the
          // largest one used; rescale the accumulators, and the probabilities computed
          // against a smaller one
          const int rgh[2] = {(8 * g) / (64 / RG), (32 + 8 * g) / (64 / RG)};
#pragma unroll
          for (int j4 = 0; j4 < NJ; j4++) {
            const int h = 16 * j4 + r16;
            float mnew = sm.wref[par][0][h];
#pragma unroll
            for (int q = 1; q < RG; q++) mnew = fmaxf(mnew, sm.wref[par][q][h]);
            if (mnew != m_ref[j4]) {
              const float alpha = __builtin_amdgcn_exp2f(m_ref[j4] - mnew);   // 0 if m_ref = -inf
#pragma unroll
              for (int k = 0; k < 8; k++) O[k][j4] *= alpha;
              l_acc[j4] *= alpha;
              m_ref[j4] = mnew;
            }
#pragma unroll
            for (int half = 0; half < 2; half++) {
              const float qh = sm.wref[par][rgh[half]][h];
              if (qh != mnew) {
                const f16 e = (f16)__builtin_amdgcn_exp2f(qh - mnew);
                bop[j4][half] *= f16x8{e, e, e, e, e, e, e, e};
              }
            }
          }
        }
#pragma unroll
        for (int j4 = 0; j4 < NJ; j4++) l_acc[j4] += sum8(bop[j4][0]) + sum8(bop[j4][1]);

        // ---- PV: O^T[128pw + 16tau + feature][head] += V^T P^T over the tile's 64 rows.
        // 4-bit transpose read: lane s of group g supplies tile row 8g+s (s < 8) or
        // 32+8g+s-8; dword 0 then holds rows 8g..8g+7 and dword 1 rows 32+8g.. of feature
        // 16*tau + r16.
        if (kFp8 && (fl & 2)) {
          // 8-bit transpose read: lane s of group g supplies 8 bytes of tile row 8g + s/2
          // (a0) or 32 + 8g + s/2 (a1) at feature offset 8*(s%2) of piece tau; lane i
          // receives feature 16*tau + i of the group's 8 rows.
          const int R0 = 8 * g + (r16 >> 1), R1 = R0 + 32;
          const SMLA_LDS uint8_t* tb0 = slot + (R0 >> 4) * F::kPortion + 16 * (R0 & 15) + 8 * (r16 & 1) + 2048 * pw;
          const SMLA_LDS uint8_t* tb1 = slot + (R1 >> 4) * F::kPortion + 16 * (R1 & 15) + 8 * (r16 & 1) + 2048 * pw;
#pragma unroll
          for (int k = 0; k < 8; k++) {
            const u32x2 d0 = lds_read_tr8(tb0 + 256 * k);
            const u32x2 d1 = lds_read_tr8(tb1 + 256 * k);
            const f16x8 a0 = fp8x8(d0.x, d0.y), a1 = fp8x8(d1.x, d1.y);
#pragma unroll
            for (int j4 = 0; j4 < NJ; j4++) {
              O[k][j4] = mfma16x16x32(a0, bop[j4][0], O[k][j4]);
              O[k][j4] = mfma16x16x32(a1, bop[j4][1], O[k][j4]);
            }
          }
        } else if (!kFp8 && (fl & 2)) {
          const int R = (r16 < 8) ? (8 * g + r16) : (32 + 8 * g + r16 - 8);
          const SMLA_LDS uint8_t* tb = slot + (R >> 4) * F::kPortion + 16 * (R & 15) + 1024 * pw;
#pragma unroll
          for (int k = 0; k < 8; k++) {
            const int tau = 8 * pw + k;
            const u32x2 d = lds_read_tr4(tb + 256 * (k >> 1) + 8 * (k & 1));
            const f16x8 sc0 = lds_load<f16x8>(&sm.sc[par][tau][8 * g]);
            const f16x8 sc1 = lds_load<f16x8>(&sm.sc[par][tau][32 + 8 * g]);
            const f16x8 a0 = unpack8_pairs(d.x, sc0), a1 = unpack8_pairs(d.y, sc1);
#pragma unroll
            for (int j4 = 0; j4 < NJ; j4++) {
              O[k][j4] = mfma16x16x32(a0, bop[j4][0], O[k][j4]);
              O[k][j4] = mfma16x16x32(a1, bop[j4][1], O[k][j4]);
            }
          }
        }

        // ---- end of a token segment: write the output or a partial, start afresh
        if (s == n || cu.ci == cpt - 1) {
          const int64_t t = cu.t;
          const int64_t tok0 = t * cpt;
          const bool full = (c_lo <= tok0) && (c_hi >= tok0 + cpt);
          const int seg = (t == t_first) ? 0 : 1;
          const int64_t slot_id = ((int64_t)hb * G + w) * 2 + seg;
#pragma unroll
          for (int j4 = 0; j4 < NJ; j4++) {
            const float Ls = wave_sum_xor16_32(l_acc[j4]);
            const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
            const float lse_nat = Ls > 0.0f ? (m_ref[j4] + log2f(Ls)) * kLn2 : -INFINITY;
            const int hl = 16 * j4 + r16;
            if (full) {
              f16* op = (f16*)A.out + (t * A.H + head0 + hl) * kLatent;
#pragma unroll
              for (int k = 0; k < 8; k++) {
                const f32x4 v = O[k][j4] * inv;
                *(f16x4*)(op + 16 * (8 * pw + k) + 4 * g) = f16x4{(f16)v.x, (f16)v.y, (f16)v.z, (f16)v.w};
              }
              if (pw == 0 && g == 0) A.lse[t * A.H + head0 + hl] = lse_nat;
            } else {
              const uint32_t po = (uint32_t)((slot_id * NH + hl) * kLatent) * 4u;
#pragma unroll
              for (int k = 0; k < 8; k++) merge_st4(ws_o, po + 4u * (16 * (8 * pw + k) + 4 * g), O[k][j4] * inv);
              if (pw == 0 && g == 0) merge_st1(ws_l, (uint32_t)(slot_id * NH + hl) * 4u, lse_nat);
            }
#pragma unroll
            for (int k = 0; k < 8; k++) O[k][j4] = f32x4{0.f, 0.f, 0.f, 0.f};
            m_ref[j4] = -INFINITY;
            l_acc[j4] = 0.0f;
          }
        }
        cu.next(cpt);
      }
      __syncthreads();
    }
  }

  // ---- publish this range's partials and merge the tokens whose last range this is.
  // The range's tokens: the first and the last may be shared with other ranges (partial),
  // every other one lies inside it.  The ring is idle from here on (every DMA has
  // completed) and serves as the merge's scratch.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (n <= 0) return;
  int64_t pend_t[2] = {-1, -1};
  {
    const int64_t t0 = c_lo / cpt, t1 = (c_hi - 1) / cpt;
    auto partial = [&](int64_t t) { return !((c_lo <= t * cpt) && (c_hi >= t * cpt + cpt)); };
    if (partial(t0)) pend_t[0] = t0;
    if (t1 != t0 && partial(t1)) pend_t[1] = t1;
  }
  constexpr int kTeamHeads = NH == 64 ? 32 : 16;   // heads merged by each active team
  const int team = tid >> 8, tt = tid & 255;
  const bool active = NH == 64 || team == 0;
  float* const scratch = (float*)sm.ring + 2048 * team;
#pragma unroll
  for (int seg = 0; seg < 2; seg++) {
    const int64_t t = pend_t[seg];
    if (t < 0) continue;
    const int64_t tok0 = t * cpt;
    const int64_t w_lo = wg_of_chunk(tok0, C, G), w_hi = wg_of_chunk(tok0 + cpt - 1, C, G);
    if (tid == 0) {
      int32_t* cnt = A.counters + (int64_t)hb * A.T + t;
      const int old = atomicAdd(cnt, 1);
      const int last = (old == (int)(w_hi - w_lo));
      if (last) atomicExch(cnt, 0);
      sm.flag = last;
    }
    __syncthreads();
    const int last = sm.flag;
    __syncthreads();
    if (!last) continue;
    // split s of token t is range w_lo + s; range w_lo holds t in slot 1 exactly when it
    // starts before the token
    const uint32_t sl0 = (uint32_t)(((int64_t)hb * G + w_lo) * 2);
    const uint32_t seg0 = (wg_first_chunk(w_lo, C, G) < tok0) ? 1u : 0u;
    const uint32_t h_off = active ? (uint32_t)(kTeamHeads * team) : 0u;
    auto part = [&](int s, uint32_t* o_off, uint32_t* l_off) {
      const uint32_t sl = sl0 + 2u * (uint32_t)s + (s == 0 ? seg0 : 0u);
      *o_off = (sl * (uint32_t)NH + h_off) * (uint32_t)(kLatent * 4);
      *l_off = (sl * (uint32_t)NH + h_off) * 4u;
    };
    lse_merge<kTeamHeads, true>((int)(w_hi - w_lo + 1), ws_o, ws_l, part,
                                (f16*)A.out + (t * A.H + head0 + h_off) * kLatent,
                                A.lse + t * A.H + head0 + h_off, scratch, tt, active);
    __syncthreads();
  }
}

hipError_t launch_decode_nvfp4_ws(const DecodeArgs& a, hipStream_t s, int heads, bool grouped) {
  const dim3 grid(a.G * a.HB), block(kThreads);
  if (grouped)
    hipLaunchKernelGGL((sparse_mla_decode_ws_kernel<64, true, false>), grid, block, 0, s, a);
  else if (heads == 64)
    hipLaunchKernelGGL((sparse_mla_decode_ws_kernel<64, false, false>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((sparse_mla_decode_ws_kernel<16, false, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_fp8_ws(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((sparse_mla_decode_ws_kernel<64, false, true>), dim3(a.G * a.HB), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace smla

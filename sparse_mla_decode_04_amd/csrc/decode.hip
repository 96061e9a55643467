// Fused sparse MLA decode over NVFP4 cache rows for gfx950 (MI355X).
//
// "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section
// "Four-bit caches make room": for every decode token the kernel loads only the cache
// rows named by the sparse indexer's 2,048-entry list, unpacks the NVFP4 values on chip
// (no FP8 staging buffer in HBM) and runs attention with FP16 operands and FP32
// accumulation; empty list entries cost no load.  The page's kernel overlaps unpacking
// with scoring and accumulation through a three-slot pipeline over warp groups and sizes
// SM clusters by the token batch.  The gfx950 design keeps the overlap and the
// batch-sized decomposition, mapped onto wave64, LDS DMA and MFMA:
//
//  * Workgroup = 4 waves, one block of 16*NG heads, one stream-K range of 64-row tiles
//    (smla_decode.hpp).  Block ids are remapped so that the head blocks of a range, and
//    neighbouring ranges, run on one XCD (shared L2).  With 16 heads a workgroup fits in
//    half of a CU's LDS, so two of them share each CU and hide each other's waits.
//  * Gather: the rows of tile i+D are fetched while tile i is computed, straight from HBM
//    into a ring of D+1 LDS slots with buffer_load ... lds (16 bytes per lane, no register
//    staging).  Wave w fetches rows 16w..16w+15 of a tile; its part of a slot is stored
//    piece-major ([16-byte piece][row]) so that the row reads of the scoring step are
//    free of bank conflicts.  Empty entries use an out-of-range buffer offset: the
//    hardware returns zeros and touches no memory.  The index list runs two tiles ahead
//    of the rows through the same DMA path, so every wait is an exact count of in-order
//    vector memory operations.
//  * QK^T: wave w scores its own 16 rows against the block's heads with
//    v_mfma_f32_16x16x32_f16 (M = rows, N = heads, K = 576 in 18 steps, in two
//    independent accumulation chains).  Each lane unpacks its row's codes straight into
//    the A operand (hardware E2M1 -> fp16 convert, times the E4M3 group scale by an exact
//    fp16 multiply) once for all NG head groups; the query stays in registers as the B
//    operand.
//  * Online softmax in fp32, base 2 (scores pre-scaled by softmax_scale*log2 e), with a
//    per-head reference maximum shared by the four waves.  A wave keeps the reference
//    unless its own rows exceed it by more than 8, in which case it uses its own maximum;
//    probabilities therefore stay <= 256 in fp16.  After the tile's barrier the new
//    reference is the largest one any wave used, and the few probabilities computed
//    against a smaller one are scaled down (rare: the reference settles after the first
//    tiles).  Empty entries get probability 0.
//  * PV: wave w owns output features 128w..128w+127 (8 tiles of 16 = one scale group
//    each) for all heads of the block over the tile's 64 rows: O^T += V^T P^T with
//    M = features, N = heads, K = rows.  V^T comes straight from the raw nibbles through
//    the LDS 4-bit transpose read (ds_read_b64_tr_b4: 16 rows of one feature per lane),
//    scaled by a per-tile fp16 table of the rows' E4M3 group scales.
//  * Epilogue: a range that covers a whole token writes out = O/l and lse directly;
//    otherwise it writes its normalized partial and LSE (device-coherent stores), and
//    after its last tile counts itself in; the last range of a token merges the partials
//    (smla_combine.hpp).
//
// One barrier per tile between each wave's QK (which fills the probability and scale
// tables and waits for its own DMA) and everyone's PV (which reads every wave's rows).  The ring slot
// refilled after the barrier of tile i was last read by the PV of tile i-1, which every
// wave has finished by then.  With a distance of one tile (two slots) a second barrier at
// the start of each tile frees the other slot, so the next tile's rows are requested a
// whole tile of work ahead.
//
// The query of the first token of a range is loaded into registers directly; the query of
// every later token is staged into LDS by the same DMA path, issued just before the rows of
// the token's first tile, and moved to registers at that tile.
//
// The same skeleton with kFp8 = true attends over 576-byte FP8 E4M3 rows, reading V^T
// through the 8-bit LDS transpose read: either the rows pass 1 of the staged variant
// wrote to HBM (one per list entry), or the rows of a pool kept in FP8 (entry v names
// pool row v, as for NVFP4).
#include "smla_launch.hpp"
#include "smla_tile.hpp"

namespace smla {

namespace {

template <bool kFp8>
struct RowFmt {
  static constexpr int kRB = kFp8 ? kHeadDim : kRowBytes;   // bytes per row in HBM
  static constexpr int kPieces = kRB / 16;                   // 36 or 22
  static constexpr int kLoads = (kPieces + 3) / 4;           // DMA per wave per tile: 9 or 6
  static constexpr int kPortion = kPieces * 256;             // LDS bytes of one wave's rows
  static constexpr int kSlot = kWaves * kPortion;            // LDS bytes of one tile
};

// Staging buffers for the query: one suffices unless the distance is two tiles and a
// token may span a single tile (then the query of the token after next would overwrite
// the one being read).
template <int NG, int ST>
constexpr int kQBufs = (ST == 3 && NG == 1) ? 2 : 1;

template <int NG, int ST, bool kFp8>
struct __attribute__((aligned(16))) Smem {
  uint8_t ring[ST][RowFmt<kFp8>::kSlot];    // [slot][wave][piece][row] 16-byte pieces
  uint8_t qst[kQBufs<NG, ST>][QFmt<NG>::kBytes];   // query staging [token parity]
  int32_t idx[2][kWaves][kWR];              // index-list DMA landing zone [tile parity][wave]
  f16 sc[2][kFp8 ? 1 : 32][kPH];            // PV scales [parity][group][tile row]
  f16 pb[2][kHeadGroup * NG][kPH];          // probabilities [parity][head][tile row]
  float wref[2][kWaves][kHeadGroup * NG];   // reference each wave used [parity][wave][head]
  int wflag[2][kWaves];                     // bit 0: wave raised a reference; bit 1: wave has a row
  int flag;
};

}  // namespace

template <int NG, int ST, bool kFp8, int WPC>
__global__ __launch_bounds__(256, WPC) void sparse_mla_decode_kernel(DecodeArgs A) {
  using F = RowFmt<kFp8>;
  constexpr int NH = kHeadGroup * NG;
  constexpr int D = ST - 1;   // prefetch distance in tiles
  constexpr int QB = kQBufs<NG, ST>;
  static_assert(D == 1 || D == 2, "ring of two or three slots");
  __shared__ Smem<NG, ST, kFp8> sm;
  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r16 = lane & 15, g = lane >> 4;

  // XCD-aware order: hardware deals block b to XCD b % 8; give each XCD a contiguous run
  // of logical workgroups (the head blocks of one range, then neighbouring ranges).
  const int nb = gridDim.x, b = blockIdx.x, xcd = b & 7, per = nb >> 3, rem = nb & 7;
  const int L = xcd * per + min(xcd, rem) + (b >> 3);
  const int w = L / A.HB, hb = L - w * A.HB;
  const int64_t C = A.tiles;
  const int G = A.G;
  const int cpt = A.cpt;
  const int64_t c_lo = wg_first_chunk(w, C, G), c_hi = wg_first_chunk(w + 1, C, G);
  const int n = (int)(c_hi - c_lo);
  const int head0 = hb * NH;
  const float sl2 = A.scale_log2;

  const i32x4 rs_rows = make_rsrc(A.rows, A.rows_bytes);
  const i32x4 rs_idx = make_rsrc(A.idx, A.idx_bytes);
  const i32x4 rs_q = make_rsrc(A.q, A.q_bytes);
  const __amdgpu_buffer_rsrc_t ws_o = merge_rsrc(A.part_o, A.part_o_bytes);
  const __amdgpu_buffer_rsrc_t ws_l = merge_rsrc(A.part_lse, A.part_lse_bytes);
  SMLA_LDS uint8_t* const ring = (SMLA_LDS uint8_t*)sm.ring;
  SMLA_LDS int32_t* const idxbuf = (SMLA_LDS int32_t*)sm.idx;

  // DMA of this wave's 16 index entries of tile cur (relative index i) into idx[i & 1][wid].
  auto issue_idx = [&](const Cursor& cur, int i) {
    const int k = cur.ci * kTileRows + kWR * wid + lane;
    const bool ok = cur.c < c_hi && k < A.topk;
    const uint32_t voff = ok ? (uint32_t)(cur.t * A.topk + k) * 4u : kOOB;
    if (lane < kWR) dma4(rs_idx, voff, lds_addr(idxbuf + ((i & 1) * kWaves + wid) * kWR));
  };
  // DMA of this wave's share of the query rows of token t into its staging buffer.
  auto issue_q = [&](int64_t t) {
    dma_q<NG>(A, rs_q, t, head0, wid, lane, lds_addr((SMLA_LDS uint8_t*)sm.qst[t % QB]));
  };
  // DMA of this wave's rows of tile cur into ring slot i % ST (its index entries must have
  // landed), preceded by the query of its token when the tile starts a token (i >= 1).
  // The slot was last read by the PV of tile i - ST, which every wave finished before the
  // barrier of tile i - D that precedes this call.  Returns the mask of valid rows (bit r =
  // wave row r).
  auto issue_rows = [&](const Cursor& cur, int i) -> uint32_t {
    if (i >= 1 && cur.ci == 0 && cur.c < c_hi) issue_q(cur.t);
    const int k = cur.ci * kTileRows + kWR * wid + r16;
    const int32_t v = idxbuf[((i & 1) * kWaves + wid) * kWR + r16];
    const bool ok = cur.c < c_hi && k < A.topk && row_valid(v, A.pool_rows);
    uint32_t base;
    if constexpr (kFp8)
      base = (uint32_t)(A.fp8_pool ? v : cur.t * A.topk + k) * (uint32_t)kHeadDim;
    else
      base = storage_row((uint32_t)v, A.map) * (uint32_t)kRowBytes;
    const uint32_t lds0 = lds_addr(ring + (i % ST) * F::kSlot + wid * F::kPortion);
#pragma unroll
    for (int kk = 0; kk < F::kLoads; kk++) {
      const int piece = 4 * kk + g;
      const uint32_t voff = ok ? base + 16u * piece : kOOB;
      // the last instruction of an NVFP4 row set covers pieces 20..23 of which 22 and 23
      // do not exist: those lanes stay idle (the instruction is still issued)
      if (4 * kk + 3 < F::kPieces || piece < F::kPieces) dma16(rs_rows, voff, lds0 + 1024u * kk);
    }
    return (uint32_t)__ballot(ok && g == 0) & 0xFFFFu;
  };

  // ---- prologue: query of the first token (into registers); index entries of tiles 0, 1;
  // then rows(d) and idx(d+2) for d < D.  From here on the vector memory operations are
  // issued in the order  ..., [q(c)], rows(c), idx(c+2), [q(c+1)], rows(c+1), ...  where
  // q(c) is the query DMA of a token whose first tile c lies in the range (c >= 1).  With
  // D = 2 the rows of tile i+2 are issued after the barrier of tile i; with D = 1 the rows
  // of tile i+1 are issued at the start of tile i, after a barrier of their own.
  QReg<NG> Q;
  Cursor cr, cx;   // cursors of the next row DMA (tile i+D) and index DMA (tile i+D+2)
  cr.init(c_lo, cpt);
  cx.init(c_lo, cpt);
  load_q<NG>(A, cr.t, head0, r16, g, Q);
  issue_idx(cx, 0);
  cx.next(cpt);
  issue_idx(cx, 1);
  cx.next(cpt);
  wait_vm<0>();
  uint32_t vmq[D + 1];   // valid-row masks of tiles i .. i+D
#pragma unroll
  for (int d = 0; d < D; d++) {
    vmq[d] = issue_rows(cr, d);
    cr.next(cpt);
    issue_idx(cx, d + 2);
    cx.next(cpt);
  }
  vmq[D] = 0;

  f32x4 O[NG][8];
  float m_ref[NG], l_acc[NG];
#pragma unroll
  for (int j = 0; j < NG; j++) {
#pragma unroll
    for (int k = 0; k < 8; k++) O[j][k] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref[j] = -INFINITY;
    l_acc[j] = 0.0f;
  }
  Cursor cu;   // tile being computed
  cu.init(c_lo, cpt);
  const int64_t t_first = cu.t;
  int64_t pend_t[2] = {-1, -1};   // tokens this range wrote partials for (first, last)

  for (int i = 0; i < n; i++) {
    const int par = i & 1;
    SMLA_LDS uint8_t* const slot = ring + (i % ST) * F::kSlot;
    if constexpr (D == 2) {
      // rows(i), idx(i+2) and a query DMA issued before rows(i+1) have landed; rows(i+1)
      // and idx(i+3) may still be in flight
      wait_vm<F::kLoads + 1>();
      // first tile of a later token: every wave waited for its share of the staged query
      // before the previous tile's barrier
      if (i > 0 && cu.ci == 0) read_q<NG>((const SMLA_LDS uint8_t*)sm.qst[cu.t % QB], r16, g, Q);
    } else {
      wait_vm<1>();   // rows(i) and a query DMA before them landed; idx(i+2) may be in flight
      // every wave's rows of tile i (and share of a staged query) have landed, and every
      // wave has finished the PV of tile i-1: the other slot is free for tile i+1, whose
      // rows are fetched now, a whole tile of work ahead of their use
      __syncthreads();
      vmq[1] = issue_rows(cr, i + 1);
      cr.next(cpt);
      issue_idx(cx, i + 3);
      cx.next(cpt);
      if (i > 0 && cu.ci == 0) read_q<NG>((const SMLA_LDS uint8_t*)sm.qst[cu.t % QB], r16, g, Q);
    }
    const uint32_t vm = vmq[0];

    // ---- QK^T: rows 16*wid + r16 of the tile (A operand) against the block's heads
    {
      const SMLA_LDS uint8_t* por = slot + wid * F::kPortion;
      f32x4 acc[2][NG];
#pragma unroll
      for (int j = 0; j < NG; j++) acc[0][j] = acc[1][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (vm != 0) {
        if constexpr (!kFp8) {
          u32x4 cw[4];
#pragma unroll
          for (int k = 0; k < 4; k++) cw[k] = lds_load<u32x4>(por + 256 * (4 * g + k) + 16 * r16);
          const u32x2 scb = lds_load<u32x2>(por + 256 * (16 + (g >> 1)) + 16 * r16 + 8 * (g & 1));
          const u32x4 rb = lds_load<u32x4>(por + 256 * (18 + g) + 16 * r16);
          const f16x2 s01 = e4m3x2<false>(scb.x), s23 = e4m3x2<true>(scb.x);
          const f16x2 s45 = e4m3x2<false>(scb.y), s67 = e4m3x2<true>(scb.y);
          const f16 sf[8] = {s01.x, s01.y, s23.x, s23.y, s45.x, s45.y, s67.x, s67.y};
#pragma unroll
          for (int k = 0; k < 16; k++) {
            const f16 s = sf[k >> 1];
            const f16x8 a = unpack8(cw[k >> 2][k & 3], f16x2{s, s});
#pragma unroll
            for (int j = 0; j < NG; j++) acc[k & 1][j] = mfma16x16x32(a, Q.v[j][k], acc[k & 1][j]);
          }
          const f16x8 r0 = fp8x8(rb.x, rb.y), r1 = fp8x8(rb.z, rb.w);
#pragma unroll
          for (int j = 0; j < NG; j++) {
            acc[0][j] = mfma16x16x32(r0, Q.v[j][16], acc[0][j]);
            acc[1][j] = mfma16x16x32(r1, Q.v[j][17], acc[1][j]);
          }
          // PV scale table: this wave's rows, empty rows scaled by zero
          const bool rv = (vm >> r16) & 1;
          const int row = kWR * wid + r16;
#pragma unroll
          for (int jj = 0; jj < 8; jj++) sm.sc[par][8 * g + jj][row] = rv ? sf[jj] : (f16)0.0f;
        } else {
#pragma unroll
          for (int k = 0; k < 8; k++) {
            const u32x4 cw = lds_load<u32x4>(por + 256 * (8 * g + k) + 16 * r16);
            const f16x8 a0 = fp8x8(cw.x, cw.y), a1 = fp8x8(cw.z, cw.w);
#pragma unroll
            for (int j = 0; j < NG; j++) {
              acc[0][j] = mfma16x16x32(a0, Q.v[j][2 * k], acc[0][j]);
              acc[1][j] = mfma16x16x32(a1, Q.v[j][2 * k + 1], acc[1][j]);
            }
          }
          const u32x4 rb = lds_load<u32x4>(por + 256 * (32 + g) + 16 * r16);
          const f16x8 r0 = fp8x8(rb.x, rb.y), r1 = fp8x8(rb.z, rb.w);
#pragma unroll
          for (int j = 0; j < NG; j++) {
            acc[0][j] = mfma16x16x32(r0, Q.v[j][16], acc[0][j]);
            acc[1][j] = mfma16x16x32(r1, Q.v[j][17], acc[1][j]);
          }
        }
      } else if constexpr (!kFp8) {
#pragma unroll
        for (int jj = 0; jj < 8; jj++) sm.sc[par][8 * g + jj][kWR * wid + r16] = (f16)0.0f;
      }

      // acc[.][j][jj] = score of tile row 16*wid + 4g + jj for head 16j + r16.  The wave's
      // reference for a head is the shared one unless its rows exceed that by more than
      // the slack, then its own maximum.
      bool raised = false;
      const int rbase = kWR * wid + 4 * g;
#pragma unroll
      for (int j = 0; j < NG; j++) {
        const f32x4 a = acc[0][j] + acc[1][j];
        float s[4];
#pragma unroll
        for (int jj = 0; jj < 4; jj++) s[jj] = ((vm >> (4 * g + jj)) & 1) ? a[jj] * sl2 : -INFINITY;
        const float mx = wave_max_xor16_32(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
        const float ref = (mx > m_ref[j] + kSlack) ? mx : m_ref[j];
        raised |= ref != m_ref[j];
        f16 p[4];
#pragma unroll
        for (int jj = 0; jj < 4; jj++)
          p[jj] = (s[jj] == -INFINITY) ? (f16)0.0f : (f16)__builtin_amdgcn_exp2f(s[jj] - ref);
        lds_store<f16x4>(&sm.pb[par][kHeadGroup * j + r16][rbase], f16x4{p[0], p[1], p[2], p[3]});
        if (g == 0) sm.wref[par][wid][kHeadGroup * j + r16] = ref;
      }
      const bool wave_raised = __ballot(raised) != 0;
      if (lane == 0) sm.wflag[par][wid] = (wave_raised ? 1 : 0) | (vm != 0 ? 2 : 0);
    }

    __syncthreads();

    // ---- prefetch (distance two): rows of tile i+2 into the slot the PV of tile i-1
    // released, index entries of tile i+4 (idx(i+2) landed with an earlier wait)
    if constexpr (D == 2) {
      vmq[2] = issue_rows(cr, i + 2);
      cr.next(cpt);
      issue_idx(cx, i + 4);
      cx.next(cpt);
    }

    // ---- probabilities of the whole tile for this lane's PV operand (rows 8g..8g+7 from
    // wave g/2, rows 32+8g.. from wave 2+g/2)
    const int fl = sm.wflag[par][0] | sm.wflag[par][1] | sm.wflag[par][2] | sm.wflag[par][3];
    f16x8 bop[NG][2];
#pragma unroll
    for (int j = 0; j < NG; j++) {
      bop[j][0] = lds_load<f16x8>(&sm.pb[par][kHeadGroup * j + r16][8 * g]);
      bop[j][1] = lds_load<f16x8>(&sm.pb[par][kHeadGroup * j + r16][32 + 8 * g]);
    }
    if (fl & 1) {
      // a wave raised its reference: the new shared reference is the largest one used;
      // rescale the accumulator and the probabilities computed against a smaller one
#pragma unroll
      for (int j = 0; j < NG; j++) {
        const int h = kHeadGroup * j + r16;
        const float r0 = sm.wref[par][0][h], r1 = sm.wref[par][1][h];
        const float r2 = sm.wref[par][2][h], r3 = sm.wref[par][3][h];
        const float mnew = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
        if (mnew != m_ref[j]) {
          const float alpha = __builtin_amdgcn_exp2f(m_ref[j] - mnew);   // 0 if m_ref = -inf
#pragma unroll
          for (int k = 0; k < 8; k++) O[j][k] *= alpha;
          l_acc[j] *= alpha;
          m_ref[j] = mnew;
        }
        const float f0 = (g >> 1) == 0 ? r0 : r1, f1 = (g >> 1) == 0 ? r2 : r3;
        if (f0 != mnew) {
          const f16 e = (f16)__builtin_amdgcn_exp2f(f0 - mnew);
          bop[j][0] *= f16x8{e, e, e, e, e, e, e, e};
        }
        if (f1 != mnew) {
          const f16 e = (f16)__builtin_amdgcn_exp2f(f1 - mnew);
          bop[j][1] *= f16x8{e, e, e, e, e, e, e, e};
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NG; j++) l_acc[j] += sum8(bop[j][0]) + sum8(bop[j][1]);

    // ---- PV: O^T[16*tau + feature][head] += V^T P^T over the tile's 64 rows
    if (fl & 2) {
      if constexpr (!kFp8) {
        // 4-bit transpose read: lane s of group g supplies tile row 8g+s (s < 8) or
        // 32+8g+s-8; dword 0 then holds rows 8g..8g+7 and dword 1 rows 32+8g.. of
        // feature 16*tau + r16.
        const int R = (r16 < 8) ? (8 * g + r16) : (32 + 8 * g + r16 - 8);
        const SMLA_LDS uint8_t* tb = slot + (R >> 4) * F::kPortion + 16 * (R & 15);
#pragma unroll
        for (int k = 0; k < 8; k++) {
          const int tau = 8 * wid + k;
          const u32x2 d = lds_read_tr4(tb + 256 * (tau >> 1) + 8 * (tau & 1));
          const f16x8 sc0 = lds_load<f16x8>(&sm.sc[par][tau][8 * g]);
          const f16x8 sc1 = lds_load<f16x8>(&sm.sc[par][tau][32 + 8 * g]);
          const f16x8 a0 = unpack8_pairs(d.x, sc0), a1 = unpack8_pairs(d.y, sc1);
#pragma unroll
          for (int j = 0; j < NG; j++) {
            O[j][k] = mfma16x16x32(a0, bop[j][0], O[j][k]);
            O[j][k] = mfma16x16x32(a1, bop[j][1], O[j][k]);
          }
        }
      } else {
        // 8-bit transpose read: lane s of group g supplies 8 bytes of tile row 8g + s/2
        // at feature offset 8*(s%2); lane i receives feature 16*tau+i of rows 8g..8g+7.
        const int R0 = 8 * g + (r16 >> 1), R1 = R0 + 32;
        const SMLA_LDS uint8_t* tb0 = slot + (R0 >> 4) * F::kPortion + 16 * (R0 & 15) + 8 * (r16 & 1);
        const SMLA_LDS uint8_t* tb1 = slot + (R1 >> 4) * F::kPortion + 16 * (R1 & 15) + 8 * (r16 & 1);
#pragma unroll
        for (int k = 0; k < 8; k++) {
          const int tau = 8 * wid + k;
          const u32x2 d0 = lds_read_tr8(tb0 + 256 * tau);
          const u32x2 d1 = lds_read_tr8(tb1 + 256 * tau);
          const f16x8 a0 = fp8x8(d0.x, d0.y), a1 = fp8x8(d1.x, d1.y);
#pragma unroll
          for (int j = 0; j < NG; j++) {
            O[j][k] = mfma16x16x32(a0, bop[j][0], O[j][k]);
            O[j][k] = mfma16x16x32(a1, bop[j][1], O[j][k]);
          }
        }
      }
    }

    // ---- end of a token segment: write the output or a partial, then start afresh
    if (i == n - 1 || cu.ci == cpt - 1) {
      const int64_t t = cu.t;
      const int64_t tok0 = t * cpt;
      const bool full = (c_lo <= tok0) && (c_hi >= tok0 + cpt);
      const int seg = (t == t_first) ? 0 : 1;
      finish_segment<NG>(A, O, m_ref, l_acc, t, full, ((int64_t)hb * G + w) * 2 + seg, head0, wid, g, r16,
                         ws_o, ws_l);
      if (!full) pend_t[seg] = t;
    }
    cu.next(cpt);
#pragma unroll
    for (int d = 0; d < D; d++) vmq[d] = vmq[d + 1];
  }

  // ---- publish this range's partials and merge the tokens whose last range this is (the
  // ring is idle from here on and serves as the merge's scratch)
  publish_and_merge<NH>(A, pend_t, hb, head0, ws_o, ws_l, &sm.flag, (float*)sm.ring);
}

__global__ __launch_bounds__(256) void sparse_mla_combine_kernel(const float* __restrict__ part_o,
                                                                 const float* __restrict__ part_lse,
                                                                 int32_t T, int32_t S, int32_t H,
                                                                 f16* __restrict__ out,
                                                                 float* __restrict__ lse) {
  __shared__ float scratch[2048];
  const int t = blockIdx.x, hg = blockIdx.y;
  const __amdgpu_buffer_rsrc_t ro = merge_rsrc(part_o, (uint32_t)((uint64_t)T * S * H * kLatent * 4));
  const __amdgpu_buffer_rsrc_t rl = merge_rsrc(part_lse, (uint32_t)((uint64_t)T * S * H * 4));
  auto part = [&](int s, uint32_t* o_off, uint32_t* l_off) {
    const uint32_t base = (uint32_t)(((int64_t)t * S + s) * H + kHeadGroup * hg);
    *o_off = base * (uint32_t)(kLatent * 4);
    *l_off = base * 4u;
  };
  lse_merge<kHeadGroup, false>(S, ro, rl, part, out + ((int64_t)t * H + kHeadGroup * hg) * kLatent,
                               lse + (int64_t)t * H + kHeadGroup * hg, scratch, (int)threadIdx.x);
}

namespace {
template <int NG, int ST, bool kFp8, int WPC>
hipError_t launch_variant(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((sparse_mla_decode_kernel<NG, ST, kFp8, WPC>), dim3(a.G * a.HB), dim3(256), 0, s, a);
  return hipGetLastError();
}
}  // namespace

int decode_wgs_per_cu(bool fp8rows, int32_t NG, int variant) {
  return (!fp8rows && NG == 1 && variant != 2) ? 2 : 1;
}

hipError_t launch_decode_nvfp4(const DecodeArgs& a, hipStream_t s, int variant) {
  if (a.HB * 4 * kHeadGroup == a.H) return launch_decode_nvfp4_ws(a, s, 64, false);
  if (a.HB * 2 * kHeadGroup == a.H) return launch_variant<2, 3, false, 1>(a, s);
  if (variant == 1) return launch_decode_nvfp4_regs(a, s);
  if (variant == 2) return launch_decode_nvfp4_ws(a, s, 16, false);
  return launch_variant<1, 2, false, 2>(a, s);
}

hipError_t launch_decode_grouped(const DecodeArgs& a, hipStream_t s) { return launch_decode_nvfp4_ws(a, s, 64, true); }

hipError_t launch_decode_fp8rows(const DecodeArgs& a, hipStream_t s) {
  if (a.HB * 4 * kHeadGroup == a.H) return launch_decode_fp8_ws(a, s);
  return (a.HB * 2 * kHeadGroup == a.H) ? launch_variant<2, 2, true, 1>(a, s)
                                        : launch_variant<1, 2, true, 1>(a, s);
}

hipError_t launch_combine(const float* part_o, const float* part_lse, int32_t T, int32_t S,
                          int32_t H, void* out, float* lse, hipStream_t s) {
  hipLaunchKernelGGL(sparse_mla_combine_kernel, dim3(T, H / kHeadGroup), dim3(256), 0, s, part_o,
                     part_lse, T, S, H, (f16*)out, lse);
  return hipGetLastError();
}

}  // namespace smla

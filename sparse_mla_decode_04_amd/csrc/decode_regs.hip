// Fused sparse MLA decode over NVFP4 cache rows for blocks of 16 heads: rows gathered into
// registers, PV of one tile overlapped with QK^T of the next (gfx950 / MI355X).
//
// "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section
// "Four-bit caches make room": per decode token, only the cache rows named by the sparse
// indexer's list are loaded, the NVFP4 values are unpacked on chip, attention runs with
// FP16 operands and FP32 accumulation, and empty list entries are handled.  The page's
// kernel overlaps unpacking with scoring and accumulation through a pipeline over warp
// groups; here each wave overlaps them itself:
//
//  * Every lane loads exactly the bytes its QK^T operand needs -- pieces 4g..4g+3 of its
//    row's E2M1 codes, its 8 group scales and its rope piece, 22 dwords -- with buffer
//    loads issued one tile ahead.  An empty entry loads from an out-of-range offset:
//    zeros, no memory access.  Index entries run two tiles ahead.
//  * QK^T for tile i runs from those registers (v_mfma_f32_16x16x32_f16, M = the wave's
//    16 rows, N = 16 heads, K = 576); the lane writes its codes once to LDS, where PV reads
//    them transposed (ds_read_b64_tr_b4).
//  * Iteration i issues PV of tile i-1 and QK^T of tile i as one straight-line block --
//    they share no data -- so the MFMA chains and unpack arithmetic of both interleave
//    and one wave keeps its VALU and matrix core busy while the other waits.  Softmax of
//    tile i and the tile's single barrier follow.  Online softmax, the scale and
//    probability tables and the split epilogue are those of the LDS-ring kernel.
//  * A range that runs into a new token stages the new query in LDS by LDS DMA, issued
//    with the rows of the tile before, and waits for it with an explicit count of the
//    row loads issued since.
#include "smla_launch.hpp"
#include "smla_tile.hpp"

namespace smla {

namespace {

constexpr int kCodePortion = 16 * 256;             // one wave's 16 rows of codes, [piece][row]
constexpr int kCodeSlot = kWaves * kCodePortion;   // one tile: 16 KB
constexpr int kRowLoads = 6;                       // buffer loads per lane per tile of rows

struct __attribute__((aligned(16))) SmemR {
  uint8_t codes[2][kCodeSlot];              // [tile parity][wave][piece][row] 16-byte pieces
  uint8_t qst[QFmt<1>::kBytes];             // staged query of the next token
  f16 sc[2][32][kPH];                       // PV scales [parity][group][tile row]
  f16 pb[2][kHeadGroup][kPH];               // probabilities [parity][head][tile row]
  float wref[2][kWaves][kHeadGroup];        // reference each wave used [parity][wave][head]
  int wflag[2][kWaves];                     // bit 0: wave raised a reference; bit 1: wave has a row
  int flag;
  int early_last;                           // kEarly: the early count of the first token completed it
};
static_assert(sizeof(SmemR) <= 81920, "two workgroups per CU");

// The bytes of one row a lane needs for its QK^T operand.
struct RowRegs {
  u32x4 cw[4];   // codes, pieces 4g .. 4g+3 (latent features 128g .. 128g+127)
  u32x2 sc;      // E4M3 scales of groups 8g .. 8g+7
  u32x4 rope;    // E4M3 rope values 16g .. 16g+15
};

__device__ __forceinline__ u32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2 ld64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ int32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

}  // namespace

// kEarly (stream-K ranges that cross tokens): a range counts itself for its first token as
// soon as that token's part ends (below).  Without it (ranges inside one token, where the
// first token is the range's only one) the loop carries no code for it.
template <bool kEarly>
__global__ __launch_bounds__(256, 2) void sparse_mla_decode_regs_kernel(DecodeArgs A) {
  constexpr int NH = kHeadGroup;
  __shared__ SmemR sm;
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
  const int row = kWR * wid + r16;   // this lane's tile row in QK^T

  const __amdgpu_buffer_rsrc_t rs_rows = merge_rsrc(A.rows, A.rows_bytes);
  const __amdgpu_buffer_rsrc_t rs_idx = merge_rsrc(A.idx, A.idx_bytes);
  const i32x4 rs_q = make_rsrc(A.q, A.q_bytes);
  const __amdgpu_buffer_rsrc_t ws_o = merge_rsrc(A.part_o, A.part_o_bytes);
  const __amdgpu_buffer_rsrc_t ws_l = merge_rsrc(A.part_lse, A.part_lse_bytes);
  SMLA_LDS uint8_t* const codes = (SMLA_LDS uint8_t*)sm.codes;
  const uint32_t qst_lds = lds_addr((SMLA_LDS uint8_t*)sm.qst);

  // Index entry of this lane's row of tile cur; 0 past the range or the list.  The tile's
  // byte offset is uniform (scalar arithmetic); the lane adds 4 bytes per row.
  auto issue_idx = [&](const Cursor& cur) -> int32_t {
    const uint32_t tile_off = (uint32_t)(cur.t * A.topk + cur.ci * kTileRows) * 4u;
    const bool ok = cur.c < c_hi && cur.ci * kTileRows + row < A.topk;
    return ld32(rs_idx, ok ? tile_off + 4u * row : kOOB);
  };
  // This lane's bytes of row v for tile cur (the code pieces at instruction offsets from one
  // lane base; a row outside the list, the range or the pool reads as zeros, scales
  // included, so an empty row scales its PV contribution by zero); returns the wave's
  // valid-row mask.  Allocation rows are below 2^24 (the pool fits the buffer range), so
  // the 24-bit multiply is exact.
  const uint32_t lane_c = 64u * g, lane_s = (uint32_t)kScaleOff + 8u * g, lane_r = (uint32_t)kRopeOff + 16u * g;
  auto issue_rows = [&](const Cursor& cur, int32_t v, RowRegs& R) -> uint32_t {
    const bool ok = cur.c < c_hi && cur.ci * kTileRows + row < A.topk && row_valid(v, A.pool_rows);
    const uint32_t vb = ok ? __umul24(storage_row((uint32_t)v, A.map), (uint32_t)kRowBytes) : kOOB;
#pragma unroll
    for (int kk = 0; kk < 4; kk++) R.cw[kk] = ld128(rs_rows, vb + lane_c + 16u * kk);
    R.sc = ld64(rs_rows, vb + lane_s);
    R.rope = ld128(rs_rows, vb + lane_r);
    return __builtin_amdgcn_readfirstlane((uint32_t)__ballot(ok && g == 0) & 0xFFFFu);
  };

  // ---- QK^T of one tile from R: scores (acc) for row 16*wid + 4g + jj, head r16; the PV
  // scale table and this wave's codes go to LDS.
  auto qk = [&](const RowRegs& R, int par, const QReg<1>& Q, f32x4 (&acc)[2]) {
    const f16x2 s01 = e4m3x2<false>(R.sc.x), s23 = e4m3x2<true>(R.sc.x);
    const f16x2 s45 = e4m3x2<false>(R.sc.y), s67 = e4m3x2<true>(R.sc.y);
    const f16 sf[8] = {s01.x, s01.y, s23.x, s23.y, s45.x, s45.y, s67.x, s67.y};
#pragma unroll
    for (int k = 0; k < 16; k++) {
      const f16 sk = sf[k >> 1];
      const f16x8 a = unpack8(R.cw[k >> 2][k & 3], f16x2{sk, sk});
      acc[k & 1] = mfma16x16x32(a, Q.v[0][k], acc[k & 1]);
    }
    acc[0] = mfma16x16x32(fp8x8(R.rope.x, R.rope.y), Q.v[0][16], acc[0]);
    acc[1] = mfma16x16x32(fp8x8(R.rope.z, R.rope.w), Q.v[0][17], acc[1]);
#pragma unroll
    for (int jj = 0; jj < 8; jj++) sm.sc[par][8 * g + jj][row] = sf[jj];   // zero for an empty row
    SMLA_LDS uint8_t* const cp = codes + par * kCodeSlot + wid * kCodePortion + 16 * r16;
#pragma unroll
    for (int kk = 0; kk < 4; kk++) lds_store<u32x4>(cp + 256 * (4 * g + kk), R.cw[kk]);
  };

  // ---- the same, refilling R with the next tile's row (lane base vb) piece by piece as
  // QK^T finishes with each piece, so the row loads of a wave trickle into the memory
  // pipeline between its matrix steps instead of queueing behind the other waves' loads.
  // The fences order each piece's last use (its MFMAs, whose results feed acc, and its
  // LDS store) before its reload, so every piece keeps one set of registers.
  auto qk_refill = [&](RowRegs& R, int par, const QReg<1>& Q, f32x4 (&acc)[2], uint32_t vb) {
    f16x2 s01 = e4m3x2<false>(R.sc.x), s23 = e4m3x2<true>(R.sc.x);
    f16x2 s45 = e4m3x2<false>(R.sc.y), s67 = e4m3x2<true>(R.sc.y);
    asm volatile("" : "+v"(s01), "+v"(s23), "+v"(s45), "+v"(s67) : : "memory");
    R.sc = ld64(rs_rows, vb + lane_s);
    const f16 sf[8] = {s01.x, s01.y, s23.x, s23.y, s45.x, s45.y, s67.x, s67.y};
    SMLA_LDS uint8_t* const cp = codes + par * kCodeSlot + wid * kCodePortion + 16 * r16;
#pragma unroll
    for (int kq = 0; kq < 4; kq++) {
#pragma unroll
      for (int k = 4 * kq; k < 4 * kq + 4; k++) {
        const f16 sk = sf[k >> 1];
        acc[k & 1] = mfma16x16x32(unpack8(R.cw[kq][k & 3], f16x2{sk, sk}), Q.v[0][k], acc[k & 1]);
      }
      lds_store<u32x4>(cp + 256 * (4 * g + kq), R.cw[kq]);
      asm volatile("" : "+v"(acc[0]), "+v"(acc[1]) : : "memory");
      R.cw[kq] = ld128(rs_rows, vb + lane_c + 16u * kq);
    }
    acc[0] = mfma16x16x32(fp8x8(R.rope.x, R.rope.y), Q.v[0][16], acc[0]);
    acc[1] = mfma16x16x32(fp8x8(R.rope.z, R.rope.w), Q.v[0][17], acc[1]);
    asm volatile("" : "+v"(acc[0]), "+v"(acc[1]) : : "memory");
    R.rope = ld128(rs_rows, vb + lane_r);
#pragma unroll
    for (int jj = 0; jj < 8; jj++) sm.sc[par][8 * g + jj][row] = sf[jj];   // zero for an empty row
  };
  // Lane base of row v for tile cur (out of range if the entry is empty) and the wave's
  // valid-row mask.
  auto row_base = [&](const Cursor& cur, int32_t v, uint32_t& vmask) -> uint32_t {
    const bool ok = cur.c < c_hi && cur.ci * kTileRows + row < A.topk && row_valid(v, A.pool_rows);
    vmask = __builtin_amdgcn_readfirstlane((uint32_t)__ballot(ok && g == 0) & 0xFFFFu);
    return ok ? __umul24(storage_row((uint32_t)v, A.map), (uint32_t)kRowBytes) : kOOB;
  };

  f32x4 O[1][8];
  float m_ref[1] = {-INFINITY}, l_acc[1] = {0.0f};
#pragma unroll
  for (int k = 0; k < 8; k++) O[0][k] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- scores -> probabilities of one tile against the running reference m_cur (-inf
  // for the first tile of a segment).  The wave's reference for a head is m_cur unless its
  // rows exceed that by more than the slack, then its own maximum.  The stores of the
  // reference and flags are issued by every lane (same value, same address): no branch,
  // so this code interleaves with the PV step of the previous tile.
  auto softmax = [&](const f32x4 (&acc)[2], uint32_t vm, int par, float m_cur) {
    // exp2(score * scale_log2 - ref) in one fma each; an invalid row enters as -inf (exp2
    // gives 0), a head with no valid row takes 0 for -ref; no mask when all rows are valid
    const f32x4 a = acc[0] + acc[1];
    float sv[4];
    const bool all_valid = vm == 0xFFFFu;
#pragma unroll
    for (int jj = 0; jj < 4; jj++) sv[jj] = (all_valid || ((vm >> (4 * g + jj)) & 1)) ? a[jj] : -INFINITY;
    const float mx = wave_max_xor16_32(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])) * sl2);
    const float ref = (mx > m_cur + kSlack) ? mx : m_cur;
    const float nref = (ref == -INFINITY) ? 0.0f : -ref;
    f16 p[4];
#pragma unroll
    for (int jj = 0; jj < 4; jj++) p[jj] = (f16)__builtin_amdgcn_exp2f(fmaf(sv[jj], sl2, nref));
    lds_store<f16x4>(&sm.pb[par][r16][kWR * wid + 4 * g], f16x4{p[0], p[1], p[2], p[3]});
    sm.wref[par][wid][r16] = ref;
    const bool wave_raised = __ballot(ref != m_cur) != 0;
    sm.wflag[par][wid] = (wave_raised ? 1 : 0) | (vm != 0 ? 2 : 0);
  };

  // ---- probabilities of a whole tile for this lane's PV operand (rows 8g..8g+7 from wave
  // g/2, rows 32+8g.. from wave 2+g/2) and the tile's flags.
  auto pv_operand = [&](int par, f16x8 (&bop)[2]) -> int {
    bop[0] = lds_load<f16x8>(&sm.pb[par][r16][8 * g]);
    bop[1] = lds_load<f16x8>(&sm.pb[par][r16][32 + 8 * g]);
    return sm.wflag[par][0] | sm.wflag[par][1] | sm.wflag[par][2] | sm.wflag[par][3];
  };
  // If a wave raised its reference, the new shared reference is the largest one used: the
  // accumulator and the probabilities computed against a smaller one are rescaled.  Then
  // the tile's probabilities join the denominator.
  auto rescale = [&](int par, int fl, f16x8 (&bop)[2]) {
    if (fl & 1) {
      const float q0 = sm.wref[par][0][r16], q1 = sm.wref[par][1][r16];
      const float q2 = sm.wref[par][2][r16], q3 = sm.wref[par][3][r16];
      const float mnew = fmaxf(fmaxf(q0, q1), fmaxf(q2, q3));
      if (mnew != m_ref[0]) {
        const float alpha = __builtin_amdgcn_exp2f(m_ref[0] - mnew);   // 0 if m_ref = -inf
#pragma unroll
        for (int k = 0; k < 8; k++) O[0][k] *= alpha;
        l_acc[0] *= alpha;
        m_ref[0] = mnew;
      }
      const float f0 = (g >> 1) == 0 ? q0 : q1, f1 = (g >> 1) == 0 ? q2 : q3;
      if (f0 != mnew) {
        const f16 e = (f16)__builtin_amdgcn_exp2f(f0 - mnew);
        bop[0] *= f16x8{e, e, e, e, e, e, e, e};
      }
      if (f1 != mnew) {
        const f16 e = (f16)__builtin_amdgcn_exp2f(f1 - mnew);
        bop[1] *= f16x8{e, e, e, e, e, e, e, e};
      }
    }
    l_acc[0] += sum8(bop[0]) + sum8(bop[1]);
  };

  // ---- PV of one tile: O^T[16*tau + feature][head] += V^T P^T over its 64 rows.  4-bit
  // transpose read: lane s of group g supplies tile row 8g+s (s < 8) or 32+8g+s-8; dword 0
  // then holds rows 8g..8g+7 and dword 1 rows 32+8g.. of feature 16*tau + r16.  An empty
  // tile has zero probabilities and scales, so it adds nothing.
  const int Rt = (r16 < 8) ? (8 * g + r16) : (32 + 8 * g + r16 - 8);
  // The LDS reads of step k+2 are issued before the arithmetic of step k (the fences keep
  // the compiler from sinking them to their use or hoisting the next step's unpack), so each
  // step's reads have two steps of unpack and matrix work to land.
  auto pv = [&](int par, const f16x8 (&bop)[2]) {
    const SMLA_LDS uint8_t* tb = codes + par * kCodeSlot + (Rt >> 4) * kCodePortion + 16 * (Rt & 15);
    auto rd = [&](int k, u32x2& d, f16x8& s0, f16x8& s1) {
      const int tau = 8 * wid + k;
      d = lds_read_tr4(tb + 256 * (tau >> 1) + 8 * (tau & 1));
      s0 = lds_load<f16x8>(&sm.sc[par][tau][8 * g]);
      s1 = lds_load<f16x8>(&sm.sc[par][tau][32 + 8 * g]);
    };
    u32x2 d0, d1;
    f16x8 p0, p1, q0, q1;   // scales of step k (p) and k+1 (q)
    rd(0, d0, p0, p1);
    rd(1, d1, q0, q1);
#pragma unroll
    for (int k = 0; k < 8; k++) {
      u32x2 dn;
      f16x8 n0, n1;
      if (k < 6) rd(k + 2, dn, n0, n1);
      asm volatile("" ::: "memory");
      f16x8 a0 = unpack8_pairs(d0.x, p0), a1 = unpack8_pairs(d0.y, p1);
      asm volatile("" : "+v"(a0), "+v"(a1));   // step k's unpack comes before step k+1's
      O[0][k] = mfma16x16x32(a0, bop[0], O[0][k]);
      O[0][k] = mfma16x16x32(a1, bop[1], O[0][k]);
      if (k < 7) {
        asm volatile("" : "+v"(d1), "+v"(q0), "+v"(q1));
        d0 = d1;
        p0 = q0;
        p1 = q1;
      }
      if (k < 6) {
        d1 = dn;
        q0 = n0;
        q1 = n1;
      }
    }
  };

  Cursor cu;   // tile whose segment end is checked next
  cu.init(c_lo, cpt);
  const int64_t t_first = cu.t;
  int64_t pend_t[2] = {-1, -1};   // tokens this range wrote partials for (first, last)
  // Early count of the first token (kEarly).  A range that starts inside a token finishes
  // that token's part in its first tiles, while the range before it finishes the token at
  // its end; counted at the end of both, the token is merged by whichever ends later, and a
  // range can end up merging two tokens one after the other.  So when the first token's
  // segment ends three or more iterations before the range's last, the range counts itself
  // for it at once: its partial's stores (issued at the end of iteration e - 1) have completed
  // at the end of iteration e, where at most that iteration's 7 loads (6 row pieces and an
  // index entry) are left in flight -- no query DMA or segment end falls there while a token
  // spans four or more tiles; the barrier orders every wave's stores, and thread 0 counts in
  // iteration e + 1, using the counter's value only at that iteration's end.  The range
  // then merges the token only if its count completed it.
  int early_wait = -1;   // iteration e, or -1
  int64_t early_t = -1;
  // ---- end of a token segment after tile cu: write the output or a partial, start afresh
  auto segment_end = [&](int i) {
    if (i == n - 1 || cu.ci == cpt - 1) {
      const int64_t t = cu.t;
      const int64_t tok0 = t * cpt;
      const bool full = (c_lo <= tok0) && (c_hi >= tok0 + cpt);
      const int seg = (t == t_first) ? 0 : 1;
      finish_segment<1>(A, O, m_ref, l_acc, t, full, ((int64_t)hb * G + w) * 2 + seg, head0, wid, g, r16,
                        ws_o, ws_l);
      if (!full) {
        if (kEarly && seg == 0 && cpt >= 4 && i <= n - 4) {
          early_wait = i + 2;
          early_t = t;
        } else {
          pend_t[seg] = t;
        }
      }
    }
    cu.next(cpt);
  };

  // ---- query staging.  With two or more tiles per token, the DMA for a later token that
  // starts at tile i+1 is issued in iteration i just before that iteration's index load and
  // row loads (kRowLoads of them), so at the top of tile i+1 waiting until at most kRowLoads
  // loads are in flight covers it.  With one tile per token the DMA is issued at the top of
  // the tile itself and waited for fully.
  const bool lead = cpt > 1;
  Cursor cq;   // tile i+1
  cq.init(c_lo + 1, cpt);
  auto stage_q = [&](int i) {
    if (lead && i + 1 < n && cq.ci == 0) dma_q<1>(A, rs_q, cq.t, head0, wid, lane, qst_lds);
    cq.next(cpt);
  };
  auto new_token_q = [&](int64_t t, QReg<1>& Q) {
    if (!lead) {
      dma_q<1>(A, rs_q, t, head0, wid, lane, qst_lds);
      wait_vm<0>();
    } else {
      wait_vm<kRowLoads>();
    }
    __syncthreads();   // every wave's share has landed
    read_q<1>((const SMLA_LDS uint8_t*)sm.qst, r16, g, Q);
  };

  // ---- prologue: query of the first token; index entries of tiles 0 and 1; rows of
  // tile 0.  The loop then issues per tile i: [query DMA], rows(i+1), idx(i+2).
  // The query comes once per workgroup by LDS DMA, issued after the rows of tile 0 (so the
  // wait for the first index entries does not cover it) and read into every wave's
  // registers from LDS: a quarter of the memory traffic of four waves loading it each.
  Cursor cr, cx;   // next row load (tile i+1) and index load (tile i+2)
  cr.init(c_lo, cpt);
  cx.init(c_lo, cpt);
  const int32_t v0 = issue_idx(cx);
  cx.next(cpt);
  int32_t IV = issue_idx(cx);   // entry of the next tile whose rows are issued
  cx.next(cpt);
  RowRegs RR;
  uint32_t vm = issue_rows(cr, v0, RR);
  cr.next(cpt);
  dma_q<1>(A, rs_q, c_lo / cpt, head0, wid, lane, qst_lds);
  wait_vm<0>();
  __syncthreads();
  QReg<1> Q;
  read_q<1>((const SMLA_LDS uint8_t*)sm.qst, r16, g, Q);

  // The fence after each QK^T ties the refill of RR to the end of QK^T (its results and
  // LDS writes come first), so the old and new contents of RR never overlap and share
  // registers, and the compiler counts the loads in flight exactly.
  // ---- tile 0: QK^T, refill, softmax, barrier
  {
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    qk(RR, 0, Q, acc);
    const uint32_t vm0 = vm;
    asm volatile("" : "+v"(acc[0]), "+v"(acc[1]) : : "memory");
    stage_q(0);
    const int32_t vr = IV;
    IV = issue_idx(cx);
    cx.next(cpt);
    vm = issue_rows(cr, vr, RR);
    cr.next(cpt);
    __builtin_amdgcn_sched_barrier(0);
    softmax(acc, vm0, 0, m_ref[0]);
    __syncthreads();
  }

  // ---- tiles 1 .. n-1.  Iteration i: QK^T(i) (the probability and flag loads of tile
  // i-1 in flight meanwhile); the rare rescale of tile i-1; then as one straight-line
  // block the refill loads, softmax(i) and PV(i-1), which share no data; the segment end of
  // tile i-1; the barrier.  softmax(i) runs against the reference the segment of tile i
  // starts from (-inf if tile i starts a token), so it need not wait for the segment end.
  // LDS parity: tile i writes codes/sc/pb[i & 1] before its barrier; PV(i-1) reads
  // [(i-1) & 1], written before barrier i-1; tile i+1 writes [(i-1) & 1] again only after
  // barrier i, which every wave passes after its PV(i-1).
  // The index load of tile i+2 is issued before the row loads of tile i+1, so the wait for
  // it at the top of iteration i+1 does not wait for them.
  for (int i = 1; i < n; i++) {
    const int par = i & 1, ppar = par ^ 1;
    const bool new_seg = cu.ci == cpt - 1;   // tile i starts a later token
    int early_old = 0;
    if (kEarly && i == early_wait + 1 && tid == 0)
      early_old = atomicAdd(A.counters + (int64_t)hb * A.T + early_t, 1);
    if (new_seg) new_token_q(cu.t + 1, Q);
    stage_q(i);
    f16x8 bop[2];
    const int fl = pv_operand(ppar, bop);
    const uint32_t vmi = vm;
    const uint32_t vb = row_base(cr, IV, vm);   // rows of tile i+1
    cr.next(cpt);
    IV = issue_idx(cx);
    cx.next(cpt);
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    // Wave priority: the two waves sharing a SIMD (from two workgroups) run QK^T at the low
    // level and softmax and PV, the stretch each workgroup's barrier waits for, at the high
    // one, so a wave that reaches its tail is issued ahead of the other's matrix work.
    __builtin_amdgcn_s_setprio(0);
    qk_refill(RR, par, Q, acc, vb);
    __builtin_amdgcn_s_setprio(1);
    rescale(ppar, fl, bop);
    softmax(acc, vmi, par, new_seg ? -INFINITY : m_ref[0]);
    pv(ppar, bop);
    __builtin_amdgcn_s_setprio(0);
    segment_end(i - 1);
    if constexpr (kEarly) {
      if (i == early_wait) wait_vm<kRowLoads + 1>();   // the first token's partial has been written
      if (i == early_wait + 1 && tid == 0) {
        const int64_t tok0 = early_t * cpt;
        const int others = (int)(wg_of_chunk(tok0 + cpt - 1, C, G) - wg_of_chunk(tok0, C, G));
        const int last = early_old == others;
        if (last) atomicExch(A.counters + (int64_t)hb * A.T + early_t, 0);
        sm.early_last = last;
      }
    }
    __syncthreads();
  }

  // ---- PV of the last tile and its segment end
  {
    f16x8 bop[2];
    const int fl = pv_operand((n - 1) & 1, bop);
    rescale((n - 1) & 1, fl, bop);
    pv((n - 1) & 1, bop);
    segment_end(n - 1);
  }

  // ---- publish this range's partials and merge the tokens whose last range this is (the
  // code slots are idle from here on and serve as the merge's scratch)
  int counted = 0;
  if (kEarly && early_wait >= 0) {   // counted in iteration early_wait + 1 < n; the loop's barriers order it
    if (sm.early_last) pend_t[0] = early_t;
    counted = 1;
  }
  publish_and_merge<NH>(A, pend_t, hb, head0, ws_o, ws_l, &sm.flag, (float*)sm.codes, counted);
}

hipError_t launch_decode_nvfp4_regs(const DecodeArgs& a, hipStream_t s) {
  // ranges inside one token (G a multiple of T) never take the early count
  if (a.T > 0 && a.G % a.T == 0)
    hipLaunchKernelGGL(sparse_mla_decode_regs_kernel<false>, dim3(a.G * a.HB), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(sparse_mla_decode_regs_kernel<true>, dim3(a.G * a.HB), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace smla

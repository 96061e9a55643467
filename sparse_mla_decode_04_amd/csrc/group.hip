// Union lists of token groups for grouped decode (gfx950 / MI355X).
//
// "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily": the decode tokens
// of one agent session attend over largely the same cache rows (the speculative and query
// tokens of a session share most of their sparse-indexer selections).  Grouped decode loads
// each row of a session once for all of its tokens; this kernel builds the per-group list
// it runs over.
//
// Group g holds tokens tpg*g .. tpg*g + tpg - 1.  Its union list is every row that some
// token of the group lists (0 <= entry < pool_rows), once, in order of first occurrence
// when the lists are read token by token, each from its first entry: the rows of token 0
// in its order, then the rows of token 1 that token 0 does not list, and so on.  An entry
// of the union is row | (members << kMemberShift), bit i of members set when token i lists
// the row.  count[g] is the union's size; entries count[g] .. U-1 are -1, and a union
// larger than U is cut after its first U entries (count[g] still says how large it was).
//
// One workgroup per group: the rows go into an LDS hash table (open addressing with linear
// probing, 16384 slots for at most 8192 entries); the member bits are OR-ed into the slot;
// then entry e of the concatenated lists is kept when its token is the lowest member of
// its row and it is the first claim of that slot, and a prefix sum over entry order gives
// its position.
#include "smla_launch.hpp"
#include "smla_device.hpp"

namespace smla {

namespace {

constexpr int kSlotsLog2 = 14;
constexpr int kSlots = 1 << kSlotsLog2;   // hash table size, twice the largest entry count
constexpr int kThreadsU = 1024;
constexpr int kPerThread = kMaxGroupEntries / kThreadsU;   // 8 entries per thread, in order

struct SmemU {
  int32_t ent[kMaxGroupEntries];  // the group's list entries, read from memory once
  int32_t key[kSlots];          // row in the slot, or -1
  uint32_t mem[kSlots / 4];     // member bits, one byte per slot
  uint32_t claim[kSlots / 32];  // slot already placed in the output
  int32_t scan[kThreadsU];
};

__device__ __forceinline__ uint32_t slot_hash(int32_t row) {
  return ((uint32_t)row * 2654435761u) >> (32 - kSlotsLog2);
}

// Slot of `row`, inserting it if absent.
__device__ __forceinline__ uint32_t insert_row(SmemU& sm, int32_t row) {
  uint32_t h = slot_hash(row);
  for (int probe = 0; probe < kSlots; probe++) {
    const int32_t old = atomicCAS(&sm.key[h], -1, row);
    if (old == -1 || old == row) return h;
    h = (h + 1) & (kSlots - 1);
  }
  return 0;   // not reached: the table is never more than half full
}

// Slot holding `row` (present).
__device__ __forceinline__ uint32_t find_row(const SmemU& sm, int32_t row) {
  uint32_t h = slot_hash(row);
  for (int probe = 0; probe < kSlots; probe++) {
    if (sm.key[h] == row) return h;
    h = (h + 1) & (kSlots - 1);
  }
  return 0;
}

}  // namespace

__global__ __launch_bounds__(kThreadsU) void group_union_kernel(const int32_t* __restrict__ idx, int32_t topk,
                                                                int32_t tpg, int64_t pool_rows, int32_t U,
                                                                int32_t* __restrict__ uni,
                                                                int32_t* __restrict__ count) {
  __shared__ SmemU sm;
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int ne = tpg * topk;   // entries of the group, <= kMaxGroupEntries
  const int32_t* lists = idx + g * tpg * (int64_t)topk;

  // the entries (coalesced, all loads in flight together), cleared table
#pragma unroll 8
  for (int e = tid; e < ne; e += kThreadsU) sm.ent[e] = lists[e];
  for (int i = tid; i < kSlots; i += kThreadsU) sm.key[i] = -1;
  for (int i = tid; i < kSlots / 4; i += kThreadsU) sm.mem[i] = 0;
  for (int i = tid; i < kSlots / 32; i += kThreadsU) sm.claim[i] = 0;
  __syncthreads();

  // ---- insert every valid entry and its token's member bit
  for (int e = tid; e < ne; e += kThreadsU) {
    const int32_t v = sm.ent[e];
    if (v < 0 || v >= pool_rows) continue;
    const uint32_t h = insert_row(sm, v);
    atomicOr(&sm.mem[h >> 2], 1u << (8 * (h & 3) + e / topk));
  }
  __syncthreads();

  // ---- keep the first occurrence of each row; thread tid owns entries kPerThread*tid .. +kPerThread-1
  uint32_t keep = 0;
  int mine = 0;
#pragma unroll 4
  for (int q = 0; q < kPerThread; q++) {
    const int e = kPerThread * tid + q;
    if (e >= ne) break;
    const int32_t v = sm.ent[e];
    if (v < 0 || v >= pool_rows) continue;
    const int tok = e / topk;
    const uint32_t h = find_row(sm, v);
    const uint32_t members = (sm.mem[h >> 2] >> (8 * (h & 3))) & 0xFFu;
    if ((members & ((1u << tok) - 1u)) != 0) continue;   // an earlier token lists the row
    const uint32_t bit = 1u << (h & 31);
    if (atomicOr(&sm.claim[h >> 5], bit) & bit) continue;   // a repeat within this token
    keep |= 1u << q;
    mine++;
  }

  // ---- positions: exclusive prefix sum of the kept counts over the threads
  sm.scan[tid] = mine;
  __syncthreads();
  for (int d = 1; d < kThreadsU; d <<= 1) {
    const int add = tid >= d ? sm.scan[tid - d] : 0;
    __syncthreads();
    sm.scan[tid] += add;
    __syncthreads();
  }
  const int total = sm.scan[kThreadsU - 1];
  int pos = sm.scan[tid] - mine;
  int32_t* out = uni + g * (int64_t)U;
  for (int q = 0; q < kPerThread; q++) {
    if (!((keep >> q) & 1u)) continue;
    const int e = kPerThread * tid + q;
    const int32_t v = sm.ent[e];
    const uint32_t h = find_row(sm, v);
    const uint32_t members = (sm.mem[h >> 2] >> (8 * (h & 3))) & 0xFFu;
    if (pos < U) out[pos] = v | (int32_t)(members << kMemberShift);
    pos++;
  }
  for (int i = total + tid; i < U; i += kThreadsU) out[i] = -1;
  if (tid == 0) count[g] = total;
}

hipError_t launch_group_union(const int32_t* idx, int32_t T, int32_t topk, int32_t tpg, int64_t pool_rows,
                              int32_t U, int32_t* uni, int32_t* count, hipStream_t s) {
  hipLaunchKernelGGL(group_union_kernel, dim3(T / tpg), dim3(kThreadsU), 0, s, idx, topk, tpg, pool_rows, U,
                     uni, count);
  return hipGetLastError();
}

}  // namespace smla

/*
 * smla.h -- C ABI of the sparse NVFP4 multi-head-latent-attention decode library
 * (libsmla.so, HIP kernels for AMD gfx950 / MI355X).
 *
 * The method: "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily",
 * section "Four-bit caches make room".  The MLA KV cache is stored as NVFP4 (four-bit
 * values with one FP8 scale per group of 16), which shrinks a cache row from 576 to
 * 352 bytes; the native sparse-attention kernel loads only the rows the sparse indexer
 * selected, unpacks them on chip, runs attention with FP16 operands and FP32
 * accumulation, handles the empty entries of the 2,048-position index list, and sizes
 * its work decomposition by the token batch.  A staged variant first unpacks NVFP4 into
 * FP8 buffers and then runs attention.
 *
 * Cache row (SMLA_ROW_BYTES = 352 bytes), one per cached token:
 *   bytes [0, 256)    512 latent values as E2M1 codes; element 2i in bits 3:0 and
 *                     element 2i+1 in bits 7:4 of byte i
 *   bytes [256, 288)  32 FP8 E4M3 (OCP "FN") scales; byte 256+j scales elements 16j..16j+15
 *   bytes [288, 352)  64 rope values as FP8 E4M3
 * A latent value is E2M1(code) * E4M3(scale); a rope value is E4M3(code).  Both are
 * exact in fp16.  The query of a head has 576 fp16 values: the first 512 pair with the
 * latent, the last 64 with the rope part; the attention output is the 512-wide latent.
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are device memory owned by the caller; the library never
 *     allocates, frees or synchronizes.  Arrays are dense, row-major, and must be
 *     16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only enqueued;
 *     completion is observed by the caller (event or stream synchronize).
 *   - Return value: SMLA_OK or a negative smla_status.  Arguments are checked on the
 *     host before anything is enqueued; on error nothing is enqueued.  No C++
 *     exception crosses this interface.
 *   - Index lists: int32, -1 (any negative value) marks an empty entry.  An entry
 *     >= pool_rows is treated as empty as well, so no list entry can make a kernel read
 *     outside the pool.
 *   - Size limit: the decode and combine kernels address each array through a buffer
 *     resource with a 32-bit byte range, so each of the query, the index lists, the
 *     cache pool (pool_rows * 352 bytes; about 12.2 million rows), the staged FP8 rows,
 *     the partial results and the workspace must stay within 0xFFFFF000 bytes, and a
 *     decode call must have fewer than 2^31 tiles of 64 list entries (T * ceil(topk/64)).
 *     A call beyond that returns SMLA_ERR_UNSUPPORTED.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define SMLA_API __attribute__((visibility("default")))
#else
#define SMLA_API
#endif

#define SMLA_ROW_BYTES 352
#define SMLA_HEAD_DIM 576
#define SMLA_LATENT_DIM 512
#define SMLA_ROPE_DIM 64
#define SMLA_GROUP 16

typedef enum {
  SMLA_OK = 0,
  SMLA_ERR_INVALID_ARG = -1,   /* null pointer, bad size, misalignment */
  SMLA_ERR_UNSUPPORTED = -2,   /* a shape the kernels do not handle (e.g. H not a multiple of 16) */
  SMLA_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
  SMLA_ERR_LAUNCH = -4,        /* the HIP runtime rejected a kernel launch */
} smla_status;

/* Human-readable name of a status code (static string). */
SMLA_API const char* smla_status_string(int status);

/*
 * Row codec, cache write ("Four-bit caches make room": NVFP4 stays the storage format).
 * Quantizes n fp16 rows src_dev[n][576] and writes each as a 352-byte cache row at
 * kv_pool_dev + slots_dev[i] * 352.  Per group of 16 latent values: scale = E4M3 nearest
 * to amax/6 (ties to even, saturating at 448); code = E2M1 nearest to x/scale (ties to
 * even, saturating at 6, sign kept; a zero scale gives signed zeros).  Rope values:
 * E4M3 nearest (ties to even, saturating at 448).  Rows whose slot is negative or
 * >= pool_rows are skipped.  Inputs must be finite.  Slots must be distinct (two rows
 * written to one slot race).  n == 0 enqueues nothing.
 */
SMLA_API int nvfp4_pack_rows(const void* src_dev, const int32_t* slots_dev, int32_t n,
                    void* kv_pool_dev, int64_t pool_rows, void* stream);

/*
 * Test / inspection export of the on-chip unpack used by the decode kernels ("Four-bit
 * caches make room": the native kernel unpacks the four-bit rows on chip; this call runs
 * that same device codec and writes its fp16 result out, so it can be compared bit for bit).
 * Decodes the cache rows rows_dev[i] (i < n) to fp16 out_dev[n][576], bit-exact
 * (latent = E2M1 * E4M3 scale, rope = E4M3).  A row id that is negative or >= pool_rows
 * gives a zero row.
 */
SMLA_API int nvfp4_unpack_rows_f16(const void* kv_pool_dev, int64_t pool_rows, const int32_t* rows_dev,
                          int32_t n, void* out_dev, void* stream);

/*
 * Sparse MLA decode ("Four-bit caches make room": loads only the selected rows, unpacks
 * on chip, FP16 operands with FP32 accumulation, empty list entries handled).
 *   q_dev        fp16 [T][H][576]
 *   kv_pool_dev  uint8 [pool_rows][352] cache rows
 *   indices_dev  int32 [T][topk] row ids, -1 = empty
 *   out_dev      fp16 [T][H][512]:  sum_j softmax_j * latent_j over the valid entries
 *   lse_dev      fp32 [T][H]:       ln sum_j exp(softmax_scale * q.k_j)
 * An entry list with no valid entry gives out = 0 and lse = -inf.  Repeated rows count
 * once per entry.  H must be a multiple of 16; 1 <= topk <= 65536.  softmax_scale must be
 * finite and > 0 (SMLA_ERR_INVALID_ARG otherwise).
 * Heads are processed in blocks per workgroup: 64 heads when H is a multiple of 64 and
 * topk > 64, else 32 when H is a multiple of 32 and topk > 64, else 16.  A larger block
 * lets one unpack of a row serve more heads.
 *   num_splits   0 = automatic (smla_choose_num_splits).  Otherwise the number of
 *                workgroups per head block that share the T*ceil(topk/64) tiles of 64
 *                list entries, in equal contiguous ranges (clamped to [1, tile count]).
 *   workspace    device scratch of at least smla_decode_workspace_bytes(T, H, topk,
 *                num_splits) bytes, zero-filled before its first use.  Every call
 *                leaves the counters it uses at zero again, so a workspace can be
 *                reused by later calls on the same stream without clearing; calls that
 *                run concurrently must not share one.  May be NULL if that size is 0.
 * The partial results of the workgroups that share a token are merged inside the same
 * launch by the workgroup that finishes last (log-sum-exp combine).
 */
SMLA_API int sparse_mla_decode(const void* q_dev, const void* kv_pool_dev, int64_t pool_rows,
                      const int32_t* indices_dev, int32_t T, int32_t H, int32_t topk,
                      float softmax_scale, void* out_dev, float* lse_dev, int32_t num_splits,
                      void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * Allocation-free variant of sparse_mla_decode, for callers that cannot allocate or pass
 * device memory for a workspace: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  Arguments, result and kernels are those of
 * sparse_mla_decode without the workspace: the split partials and merge counters live in
 * a scratch array inside the library, SMLA_NOALLOC_SCRATCH_BYTES on each GPU, held until
 * the process ends.  The call allocates nothing; it clears the counters it uses with a
 * small kernel on `stream` before the decode.
 * A shape whose split work needs more scratch than that (smla_decode_workspace_bytes
 * above the limit) returns SMLA_ERR_WORKSPACE; pass a smaller num_splits or use
 * sparse_mla_decode with a workspace.  All calls on one GPU share its scratch: calls that
 * overlap on one GPU (concurrent streams, or threads) race and give wrong results; calls
 * on one stream, one after another, are safe.
 */
#define SMLA_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)
SMLA_API int sparse_mla_decode_noalloc(const void* q_dev, const void* kv_pool_dev, int64_t pool_rows,
                                       const int32_t* indices_dev, int32_t T, int32_t H, int32_t topk,
                                       float softmax_scale, void* out_dev, float* lse_dev, int32_t num_splits,
                                       void* stream);

/*
 * The split count the automatic mode of sparse_mla_decode uses for this shape on the
 * current device ("Four-bit caches make room": the kernel sizes its groups of
 * multiprocessors by the token batch; here the work decomposition is sized by T):
 * with fewer (token, head block) pairs than compute units, every token
 * is cut into the same number of tile-aligned ranges so that about one workgroup runs
 * per compute unit; otherwise the workgroups that fit the device at once share the tiles
 * (at least two tiles each).  Queries the current device's compute-unit count.
 * Returns 0 for T == 0 or a shape sparse_mla_decode rejects.
 */
SMLA_API int32_t smla_choose_num_splits(int32_t T, int32_t H, int32_t topk);

/*
 * Workspace bytes sparse_mla_decode needs (num_splits as passed to it, 0 = automatic):
 * the partial results and counters of the batch-sized split work ("Four-bit caches make
 * room", the sizing by token batch).
 * The same size serves sparse_mla_decode_fp8rows and sparse_mla_decode_fp8pool with the
 * same arguments (they pick the head blocks and the automatic split count alike).
 */
SMLA_API size_t smla_decode_workspace_bytes(int32_t T, int32_t H, int32_t topk, int32_t num_splits);

/*
 * Log-sum-exp combine of split results ("Four-bit caches make room": the merge step that
 * the batch-sized split of each token's index list implies; the decode runs the same merge
 * inside its own launch, and this call exposes it for partials made elsewhere).
 *   partial_out_dev  fp32 [T][S][H][512]  normalized output of each split
 *   partial_lse_dev  fp32 [T][S][H]       natural-log LSE of each split (-inf = empty split)
 *   out_dev fp16 [T][H][512], lse_dev fp32 [T][H]:
 *       lse = ln sum_s exp(lse_s);  out = sum_s exp(lse_s - lse) * out_s
 * Splits with lse_s = -inf weigh zero; if all are -inf, out = 0 and lse = -inf.
 */
SMLA_API int sparse_mla_combine(const float* partial_out_dev, const float* partial_lse_dev, int32_t T,
                       int32_t S, int32_t H, void* out_dev, float* lse_dev, void* stream);

/*
 * Staged variant, pass 1 ("Four-bit caches make room": the staged implementation first
 * unpacked NVFP4 values into FP8 buffers).  For every list entry (t, j) writes the 576
 * values of row indices_dev[t][j], re-encoded as FP8 E4M3 (nearest, ties to even,
 * saturating at 448), to staged_dev + (t*topk + j)*576; an empty entry writes 576 zero
 * bytes.  staged_dev holds T*topk*576 bytes.
 */
SMLA_API int nvfp4_stage_fp8(const void* kv_pool_dev, int64_t pool_rows, const int32_t* indices_dev,
                    int32_t T, int32_t topk, void* staged_dev, void* stream);

/*
 * Staged variant, pass 2: attention over the FP8 rows written by nvfp4_stage_fp8
 * (E4M3 -> fp16 exactly, FP16 operands, FP32 accumulation).  indices_dev only marks
 * which entries are empty.  Arguments otherwise as in sparse_mla_decode, with
 * smla_decode_workspace_bytes giving the workspace size; heads are processed in blocks of
 * 64, 32 or 16 as there.
 */
SMLA_API int sparse_mla_decode_fp8rows(const void* q_dev, const void* staged_dev,
                              const int32_t* indices_dev, int64_t pool_rows, int32_t T, int32_t H,
                              int32_t topk, float softmax_scale, void* out_dev, float* lse_dev,
                              int32_t num_splits, void* workspace_dev, size_t workspace_bytes,
                              void* stream);

/*
 * FP8 cache rows, writer ("Four-bit caches make room": before NVFP4 a cache row was 576
 * bytes of FP8).  Encodes n fp16 rows src_dev[n][576] and writes each as a 576-byte row
 * at fp8_pool_dev + slots_dev[i] * 576: byte k = E4M3 code of value k (nearest, ties to
 * even, saturating at 448, sign kept).  Rows whose slot is negative or >= pool_rows are
 * skipped.  Inputs must be finite.  Slots must be distinct (two rows written to one slot
 * race).  n == 0 enqueues nothing.
 */
SMLA_API int fp8_pack_rows(const void* src_dev, const int32_t* slots_dev, int32_t n, void* fp8_pool_dev,
                           int64_t pool_rows, void* stream);

/*
 * Sparse MLA decode over a pool kept in that FP8 format: the capacity-for-latency trade
 * the same section describes (576 instead of 352 bytes per row, no unpack beyond
 * E4M3 -> fp16, which is exact).  fp8_pool_dev is uint8 [pool_rows][576] as written by
 * fp8_pack_rows; indices_dev names its rows as for sparse_mla_decode (-1 or >= pool_rows
 * = empty).  Every other argument, the result and the workspace rule are those of
 * sparse_mla_decode (smla_decode_workspace_bytes gives the size); heads are processed in
 * blocks of 64, 32 or 16 as there.  pool_rows * 576 may be at most 4 GiB - 4 KiB, else
 * SMLA_ERR_UNSUPPORTED.
 */
SMLA_API int sparse_mla_decode_fp8pool(const void* q_dev, const void* fp8_pool_dev, int64_t pool_rows,
                                       const int32_t* indices_dev, int32_t T, int32_t H, int32_t topk,
                                       float softmax_scale, void* out_dev, float* lse_dev, int32_t num_splits,
                                       void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * Sparse indexer, selection step ("Four-bit caches make room": the indexer picks the
 * 2,048 context positions per decode token whose rows the decode kernel loads; the page
 * gives no internals of its scoring, so the scores are an input here).
 *   scores_dev      float32 [T][ld]: token t's scores at positions 0 .. lengths[t] - 1
 *                   (the rest of the row is not read).  Not NaN.
 *   lengths_dev     int32 [T], each clamped to [0, ld]; NULL = every token has ld positions
 *   row_offset_dev  int32 [T]; NULL = 0
 *   out_dev         int32 [T][k]: the k positions with the largest scores, equal scores
 *                   (-0 equals +0) going to the lower position, as row_offset[t] + position
 *                   in ascending position order; a token with fewer than k positions lists
 *                   them all, then -1.  Entries must fit int32.
 *   parts           workgroups per token: 0 = chosen by the library, 1 = one (no workspace),
 *                   2 .. 64 = the token's positions split over that many (needs a workspace;
 *                   T <= 65535).  The result does not depend on it.
 *   workspace_dev   device scratch of smla_indexer_workspace_bytes(T, ld, k, parts) bytes,
 *                   16-byte aligned, zero-filled before its first use and left so by every
 *                   call; NULL runs one workgroup per token (parts 0 or 1).  Calls that share
 *                   a workspace must not overlap.
 * 1 <= k <= 65536; ld >= 0 a multiple of 4, below 2^31; scores_dev 16-byte aligned (may be
 * NULL when ld == 0).  SMLA_ERR_WORKSPACE when a split is asked for without a large enough
 * workspace.
 */
SMLA_API int sparse_indexer_topk(const float* scores_dev, int64_t ld, const int32_t* lengths_dev,
                                 const int32_t* row_offset_dev, int32_t T, int32_t k, int32_t* out_dev,
                                 int32_t parts, void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes of sparse_indexer_topk for these arguments (0: it runs one workgroup per
 * token and needs none, or the arguments are invalid).  With few tokens the library splits
 * every token's positions over several workgroups so that the selection fills the GPU
 * ("Four-bit caches make room": the decomposition is sized by the token batch).
 */
SMLA_API size_t smla_indexer_workspace_bytes(int32_t T, int64_t ld, int32_t k, int32_t parts);

/*
 * Grouped decode, step 1: union lists of token groups.  "Prime Intellect Launches Prime
 * Inference, Serving 600B Tokens Daily" (sections on the agent workload and on the
 * four-bit caches): the decode tokens of one agent session select largely the same cache
 * rows, so a session's rows can be loaded once for all of its tokens.
 *   indices_dev  int32 [T][topk] per-token lists as for sparse_mla_decode (negative or
 *                >= pool_rows = empty).  No list may name a row twice (the union counts a
 *                (row, token) pair once).
 *   tpg          tokens per group, 1..4; T % tpg == 0.  Group g is tokens tpg*g .. +tpg-1.
 *   U            capacity of a union list (entries per group).
 *   union_dev    int32 [T/tpg][U] out: the rows some token of the group lists, each once,
 *                in order of first occurrence reading the group's lists token by token;
 *                entry = row | members << 27 (bit i of members: token i lists the row);
 *                entries past the union's size are -1.
 *   count_dev    int32 [T/tpg] out: the union's size.  A union larger than U keeps its
 *                first U entries; count still reports the full size.
 * Requires tpg * topk <= 8192 and pool_rows <= 2^27 (SMLA_ERR_UNSUPPORTED otherwise).
 * Deterministic for lists without repeated rows.
 */
SMLA_API int smla_group_union(const int32_t* indices_dev, int32_t T, int32_t topk, int32_t tpg,
                              int64_t pool_rows, int32_t U, int32_t* union_dev, int32_t* count_dev,
                              void* stream);

/*
 * Grouped decode, step 2: sparse MLA decode of T tokens over the union lists of their
 * groups.  Each cache row is gathered and unpacked once per group and applied to the heads
 * of every token of the group; a score counts only where that token lists the row, so the
 * result is that of sparse_mla_decode on the tokens' own lists (for lists without repeated
 * rows), up to summation order.
 *   q_dev, out_dev, lse_dev as in sparse_mla_decode ([T][H][576], [T][H][512], [T][H]).
 *   union_dev    int32 [T/tpg][U] from smla_group_union (or any lists of that form).
 *   tpg * H must be 64 (e.g. 4 tokens of 16 heads); pool_rows <= 2^27.
 *   num_splits   0 = automatic; else workgroups sharing the (group, tile) sequence.
 *   workspace    at least smla_decode_grouped_workspace_bytes(T, H, tpg, U, num_splits)
 *                bytes, zero-filled before first use; left clean by every call.
 */
SMLA_API int sparse_mla_decode_grouped(const void* q_dev, const void* kv_pool_dev, int64_t pool_rows,
                                       const int32_t* union_dev, int32_t T, int32_t H, int32_t tpg,
                                       int32_t U, float softmax_scale, void* out_dev, float* lse_dev,
                                       int32_t num_splits, void* workspace_dev, size_t workspace_bytes,
                                       void* stream);

/* Workspace bytes sparse_mla_decode_grouped needs (0 for a shape it rejects, or T == 0). */
SMLA_API size_t smla_decode_grouped_workspace_bytes(int32_t T, int32_t H, int32_t tpg, int32_t U,
                                                    int32_t num_splits);

/*
 * Block-major multi-layer cache ("Prime Intellect Launches Prime Inference, Serving 600B
 * Tokens Daily", section on the BLHNC layout: the data of several layers is stored together
 * for each block, so that one block of every layer is one contiguous piece and moving a
 * request's cache needs one transfer per block rather than one per block and layer).
 * The layout (a cache row has no head axis, so within a block a layer's rows follow one
 * another):
 *   pool_dev  uint8 [pool_blocks][layers][block_rows][352]
 *   row v of layer l is allocation row ((v / block_rows) * layers + l) * block_rows
 *   + v % block_rows.  Each layer has pool_blocks * block_rows rows.
 * block_rows is a power of two, 1 .. 65536; layers >= 1 with layers * block_rows < 2^24;
 * 0 <= layer < layers.  A malformed layout returns SMLA_ERR_INVALID_ARG.
 */

/*
 * Cache write of layer `layer` into a block-major pool: nvfp4_pack_rows with slots_dev
 * naming rows of that layer (0 .. pool_blocks * block_rows - 1; negative or past the end =
 * skipped, slots distinct).  The row bytes are those nvfp4_pack_rows writes.
 * pool_blocks * block_rows must fit int32 (SMLA_ERR_UNSUPPORTED otherwise).
 */
SMLA_API int nvfp4_pack_rows_blhnc(const void* src_dev, const int32_t* slots_dev, int32_t n,
                                   void* pool_dev, int64_t pool_blocks, int32_t layers, int32_t layer,
                                   int32_t block_rows, void* stream);

/*
 * Sparse MLA decode of layer `layer` of a block-major pool: indices_dev names rows of that
 * layer (negative or >= pool_blocks * block_rows = empty), and every other argument, the
 * result and the workspace rule are those of sparse_mla_decode (smla_decode_workspace_bytes
 * gives the size).  The result equals sparse_mla_decode over the layer's rows laid out one
 * after another.  The whole allocation, pool_blocks * layers * block_rows * 352 bytes, must
 * stay within 0xFFFFF000 bytes (about 12.2 million rows over all layers), else
 * SMLA_ERR_UNSUPPORTED.
 */
SMLA_API int sparse_mla_decode_blhnc(const void* q_dev, const void* pool_dev, int64_t pool_blocks,
                                     int32_t layers, int32_t layer, int32_t block_rows,
                                     const int32_t* indices_dev, int32_t T, int32_t H, int32_t topk,
                                     float softmax_scale, void* out_dev, float* lse_dev, int32_t num_splits,
                                     void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * Block transfer: copies n segments of block_bytes bytes, segment src_ids_dev[i] of src_dev
 * (src_blocks segments) to segment dst_ids_dev[i] of dst_dev (dst_blocks segments).  With
 * block_bytes = layers * block_rows * 352 a segment is one block of a block-major pool, every
 * layer; gathering a request's blocks into a contiguous send buffer passes dst_ids_dev =
 * NULL (segment i), scattering a received buffer into free blocks passes src_ids_dev = NULL.
 * The copy of a layer-major cache is the same call with block_bytes = block_rows * 352 and
 * one segment per block and layer.
 *   A pair whose source or destination id is negative or past its array is skipped.
 *   Destination segments must not overlap each other or any source segment.
 *   block_bytes > 0, a multiple of 16 and below 2^36; the pointers 16-byte aligned, id
 *   arrays 4-byte aligned; n * ceil(block_bytes / 16384) < 2^24 (SMLA_ERR_UNSUPPORTED
 *   otherwise).  Device memory on both sides; n == 0 enqueues nothing.
 */
SMLA_API int blhnc_copy_blocks(const void* src_dev, int64_t src_blocks, const int32_t* src_ids_dev,
                               void* dst_dev, int64_t dst_blocks, const int32_t* dst_ids_dev, int32_t n,
                               int64_t block_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */

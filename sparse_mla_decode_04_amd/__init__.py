"""Sparse NVFP4 multi-head-latent-attention decode for MI355X (gfx950).

The hot path lives in libsmla.so (hand-written HIP kernels behind the C ABI of
include/smla.h); `binding` exposes its entry points under the same names with
torch tensors as device memory.  `workloads` draws the seeded synthetic inputs.
"""

from .binding import (  # noqa: F401
    EXPORTS, LIB_PATH, SmlaError, lib, nvfp4_pack_rows, nvfp4_unpack_rows_f16, sparse_mla_decode,
    sparse_mla_combine, nvfp4_stage_fp8, sparse_mla_decode_fp8rows, choose_num_splits,
    decode_workspace_bytes, make_workspace, group_union, sparse_mla_decode_grouped, grouped_workspace_bytes,
    make_grouped_workspace, fp8_pack_rows, sparse_mla_decode_fp8pool, sparse_indexer_topk,
    nvfp4_pack_rows_blhnc, sparse_mla_decode_blhnc, blhnc_copy_blocks, sparse_mla_decode_noalloc,
    indexer_workspace_bytes, make_indexer_workspace,
)

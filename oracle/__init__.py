"""Reference oracle for sparse NVFP4 MLA decode.  TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct CPU statement of what the
GPU path computes.  It exists so that tests, the smoke check and the CPU
baseline leg of the benchmark can compare the HIP kernels against it.  Nothing
in the product path (the C-ABI library or its Python binding) may import or
call it, and it imports nothing from the product path: the two share no code.

Sources (the web pages describing the method):
  * "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily",
    section "Four-bit caches make room": the KV cache of multi-head latent
    attention is stored as NVFP4 (4-bit values with one FP8 scale per group
    of 16), shrinking a cache row from 576 to 352 bytes; the native
    sparse-attention kernel loads only the rows chosen by the sparse indexer,
    unpacks them on chip, computes with FP16 operands and FP32 accumulation,
    and handles empty entries of the 2,048-position index list; a staged
    variant first unpacks into FP8 buffers and then runs attention.
  * "Prime Inference: Fast, Reliable Serving for Frontier Open Models",
    section "Technical deep dive" (names the NVFP4 KV compression work; the
    text of that section is not part of the page as captured).

Precision: every floating-point step is done in float64 from exactly decoded
inputs, so the oracle's results are the exact real-number results rounded
once at the end (to fp16 for outputs).

Modules:
  formats   -- E2M1 / E4M3 code tables, the NVFP4 row quantizer (pack) and
               dequantizer (unpack), the FP8 staging quantizer, the 576-byte
               FP8 row writer and reader.
  attention -- sparse MLA decode over an index list, the log-sum-exp merge of
               partial results, the staged FP8-row variant, and decode over a
               pool of 576-byte FP8 rows.
  grouping  -- union lists of token groups and decode over them (the tokens of
               one agent session sharing most of their rows).
  indexer   -- the sparse indexer's top-k selection over given scores (the step
               that produces the index lists).
  layout    -- the block-major multi-layer pool layout (blocks of every layer kept
               together), block transfers, and decode of one layer of such a pool.

Every function is pinned by tests under tests/ (test_oracle_*.py) against
values that do not come from the oracle itself: hand-typed format tables,
torch's float8_e4m3fn casts, exact rational brute force, torch's scaled dot
product attention in float64, and closed-form identities.
"""

from .formats import (  # noqa: F401
    ROW_BYTES, FP8_ROW_BYTES, LATENT_DIM, ROPE_DIM, HEAD_DIM, GROUP, CODE_BYTES, SCALE_BYTES, ROPE_BYTES,
    e2m1_value, e4m3_value, e2m1_table, e4m3_table,
    e4m3_encode, e4m3_encode_scaled_by, e2m1_encode,
    nvfp4_pack_rows_ref, nvfp4_unpack_rows_ref, fp8_stage_rows_ref,
    fp8_pack_rows_ref, fp8_unpack_rows_ref,
)
from .attention import (  # noqa: F401
    sparse_mla_decode_ref, lse_combine_ref, sparse_mla_decode_fp8rows_ref, dense_rows_for,
    sparse_mla_decode_fp8pool_ref,
)
from .grouping import group_union_ref, sparse_mla_decode_grouped_ref  # noqa: F401
from .indexer import topk_indices_ref  # noqa: F401
from .layout import (  # noqa: F401
    blocked_pool_ref, layer_rows_ref, storage_row_ref, copy_blocks_ref, sparse_mla_decode_blhnc_ref,
)

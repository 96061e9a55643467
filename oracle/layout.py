"""Block-major multi-layer pool layout.  TEST INFRASTRUCTURE ONLY (see package doc).

"Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", the section on the
BLHNC layout: the cache is laid out block-major, the data of several layers stored
together for each block, so that one block of every layer moves as one transfer instead
of one per layer.

Readings taken where the page leaves the step open:
  * A transfer moves whole blocks: with the block-major layout one block of every layer is
    one contiguous segment of L * B * 352 bytes; a layer-major cache needs one segment of
    B * 352 bytes per block and layer.  On one GPU the transfer is the copy of those
    segments into (or out of) a contiguous buffer.
  * A multi-head-latent-attention cache row has no head axis (one latent per token), so
    the layout is [block][layer][row in block][352 bytes]: row v of layer l is stored at
    row ((v // B) * L + l) * B + v % B of the allocation.
  * Decode over layer l of such a pool is decode over that layer's rows; the layout only
    moves bytes.
"""

import numpy as np

from .attention import sparse_mla_decode_ref
from .formats import ROW_BYTES


def blocked_pool_ref(layer_pools, block_rows):
    """uint8 [L, N, 352] layer-major pools (N a multiple of block_rows) -> uint8
    [N / block_rows, L, block_rows, 352] block-major pool."""
    layer_pools = np.asarray(layer_pools)
    if layer_pools.dtype != np.uint8 or layer_pools.ndim != 3 or layer_pools.shape[2] != ROW_BYTES:
        raise ValueError("layer_pools must be uint8 [L, N, 352]")
    L, N, _ = layer_pools.shape
    if N % block_rows:
        raise ValueError("N must be a multiple of block_rows")
    out = np.empty((N // block_rows, L, block_rows, ROW_BYTES), dtype=np.uint8)
    for b in range(N // block_rows):          # block b of every layer, one after another
        for l in range(L):
            out[b, l] = layer_pools[l, b * block_rows:(b + 1) * block_rows]
    return out


def layer_rows_ref(blocked, layer):
    """Rows of layer `layer` (uint8 [N, 352]) from a block-major pool."""
    blocked = np.asarray(blocked)
    nb, L, B, _ = blocked.shape
    return np.concatenate([blocked[b, layer] for b in range(nb)], axis=0) if nb else \
        np.zeros((0, ROW_BYTES), dtype=np.uint8)


def storage_row_ref(v, layer, layers, block_rows):
    """Row of the allocation that holds row v of layer `layer`."""
    return ((v // block_rows) * layers + layer) * block_rows + v % block_rows


def copy_blocks_ref(src, dst, src_ids=None, dst_ids=None, n=None):
    """Segment copy: for i < n, dst[dst_ids[i]] = src[src_ids[i]] (None = i), skipping a pair
    whose source or destination id is negative or past its array.  src and dst are arrays
    whose first axis counts segments; dst is modified in place and returned."""
    if n is None:
        n = len(src_ids) if src_ids is not None else len(dst_ids) if dst_ids is not None else len(src)
    for i in range(n):
        s = int(src_ids[i]) if src_ids is not None else i
        d = int(dst_ids[i]) if dst_ids is not None else i
        if 0 <= s < len(src) and 0 <= d < len(dst):
            dst[d] = src[s]
    return dst


def sparse_mla_decode_blhnc_ref(q, blocked, layer, indices, softmax_scale, tokens=None):
    """Decode of layer `layer` of a block-major pool: the decode over that layer's rows."""
    return sparse_mla_decode_ref(q, layer_rows_ref(blocked, layer), indices, softmax_scale, tokens=tokens)

"""Pins of the oracle's block-major multi-layer pool layout against a hand-worked example,
the storage-row formula checked row by row, and the inverse (every layer's rows back)."""

import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blocked_layout_example.json")


def _tagged(L, N):
    """Layer-major pools whose row (l, v) is filled with a byte pattern naming l and v."""
    pools = np.zeros((L, N, 352), dtype=np.uint8)
    for l in range(L):
        for v in range(N):
            pools[l, v, 0], pools[l, v, 1], pools[l, v, 2] = l, v & 255, v >> 8
            pools[l, v, 3:] = (7 * l + 3 * v) & 255
    return pools


def test_blocked_layout_matches_hand_worked_example():
    ex = json.load(open(GOLDEN))
    L, N, B = ex["layers"], ex["rows"], ex["block_rows"]
    flat = oracle.blocked_pool_ref(_tagged(L, N), B).reshape(-1, 352)
    got = [[int(r[0]), int(r[1]) + 256 * int(r[2])] for r in flat]
    assert got == ex["allocation_order"]
    assert oracle.storage_row_ref(3, 1, L, B) == ex["storage_row_of_layer1_row3"]


def test_storage_row_formula_places_every_row():
    for L, N, B in ((1, 8, 8), (3, 64, 4), (5, 96, 32), (2, 16, 1)):
        pools = _tagged(L, N)
        flat = oracle.blocked_pool_ref(pools, B).reshape(-1, 352)
        for l in range(L):
            for v in range(N):
                assert np.array_equal(flat[oracle.storage_row_ref(v, l, L, B)], pools[l, v])


def test_layer_rows_invert_the_layout():
    rng = np.random.default_rng(5)
    pools = rng.integers(0, 256, size=(4, 128, 352), dtype=np.uint8)
    blocked = oracle.blocked_pool_ref(pools, 16)
    assert blocked.shape == (8, 4, 16, 352)
    for l in range(4):
        assert np.array_equal(oracle.layer_rows_ref(blocked, l), pools[l])


def test_block_transfer_matches_hand_worked_example():
    """One block of every layer is one segment; the layer-major cache needs one per layer."""
    ex = json.load(open(GOLDEN))
    L, N, B = ex["layers"], ex["rows"], ex["block_rows"]
    pools = _tagged(L, N)
    blocked = oracle.blocked_pool_ref(pools, B)                      # [N/B, L, B, 352]
    send = np.zeros((1, L, B, 352), dtype=np.uint8)
    oracle.copy_blocks_ref(blocked, send, src_ids=[1])
    got = [[int(r[0]), int(r[1]) + 256 * int(r[2])] for r in send.reshape(-1, 352)]
    assert got == ex["block1_segment_order"]
    # the same rows from the layer-major pools: segment (block 1, layer l) = pools[l, 2:4]
    segs = pools.reshape(L, N // B, B, 352).reshape(L * (N // B), B, 352)   # segment l * nb + b
    lm = np.zeros((ex["layer_major_segments_for_block1"], B, 352), dtype=np.uint8)
    oracle.copy_blocks_ref(segs, lm, src_ids=[l * (N // B) + 1 for l in range(L)])
    assert np.array_equal(lm.reshape(-1, 352), send.reshape(-1, 352))


def test_block_copy_skips_out_of_range_pairs_and_round_trips():
    rng = np.random.default_rng(9)
    src = rng.integers(0, 256, size=(6, 2, 4, 352), dtype=np.uint8)
    dst = np.full((5, 2, 4, 352), 7, dtype=np.uint8)
    oracle.copy_blocks_ref(src, dst, src_ids=[5, -1, 2, 6, 0], dst_ids=[0, 1, 9, 3, 4])
    assert np.array_equal(dst[0], src[5]) and np.array_equal(dst[4], src[0])
    assert (dst[1] == 7).all() and (dst[2] == 7).all() and (dst[3] == 7).all()
    # gather a request's blocks into a send buffer, scatter them into other free blocks
    ids = [4, 1, 3]
    send = np.zeros((3, 2, 4, 352), dtype=np.uint8)
    oracle.copy_blocks_ref(src, send, src_ids=ids)
    back = np.zeros_like(src)
    oracle.copy_blocks_ref(send, back, dst_ids=[0, 2, 5])
    for i, b in enumerate(ids):
        assert np.array_equal(back[[0, 2, 5][i]], src[b])


def test_blocked_decode_is_decode_over_the_layer():
    """Decode of layer l of a block-major pool equals the decode over pool l on its own."""
    rng = np.random.default_rng(11)
    L, N, B, T, H, K = 3, 64, 8, 2, 16, 24
    src = rng.standard_normal((L, N, 576)).astype(np.float16)
    pools = np.stack([oracle.nvfp4_pack_rows_ref(src[l]) for l in range(L)])
    blocked = oracle.blocked_pool_ref(pools, B)
    q = rng.standard_normal((T, H, 576)).astype(np.float16)
    idx = np.stack([rng.permutation(N)[:K] for _ in range(T)]).astype(np.int32)
    idx[1, -5:] = -1
    for l in range(L):
        o1, s1 = oracle.sparse_mla_decode_blhnc_ref(q, blocked, l, idx, 1 / 24)
        o2, s2 = oracle.sparse_mla_decode_ref(q, pools[l], idx, 1 / 24)
        assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16)) and np.array_equal(s1, s2)
    # and the layers differ (the map does not collapse them onto one)
    o0, _ = oracle.sparse_mla_decode_blhnc_ref(q, blocked, 0, idx, 1 / 24)
    o2, _ = oracle.sparse_mla_decode_blhnc_ref(q, blocked, 2, idx, 1 / 24)
    assert not np.array_equal(o0, o2)

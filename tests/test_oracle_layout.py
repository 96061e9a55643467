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

"""Pins of the oracle's grouped decode (union lists of token groups, decode over them)
against a hand-worked example, numpy's set routines and the per-token decode."""

import json
import os

import numpy as np
import pytest

import oracle
from sparse_mla_decode_04_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "group_union_example.json")


def test_union_matches_hand_worked_example():
    ex = json.load(open(GOLDEN))
    union, count = oracle.group_union_ref(np.array(ex["indices"], dtype=np.int32), ex["tpg"], ex["pool_rows"],
                                          ex["U"])
    assert union.tolist() == ex["union"]
    assert count.tolist() == ex["count"]


def _random_lists(T, K, N, shared, empty_frac, seed):
    """T lists of K distinct rows each from [0, N); consecutive groups of 4 tokens share a
    fraction `shared` of their rows; some entries empty or out of range."""
    rng = np.random.default_rng(seed)
    idx = np.empty((T, K), dtype=np.int32)
    for g in range(0, T, 4):
        common = rng.choice(N, size=int(shared * K), replace=False)
        for t in range(g, min(g + 4, T)):
            rest = np.setdiff1d(np.arange(N), common)
            own = rng.choice(rest, size=K - len(common), replace=False)
            idx[t] = rng.permutation(np.concatenate([common, own]))
    idx[rng.random(idx.shape) < empty_frac] = -1
    idx[rng.random(idx.shape) < 0.02] = N + 3      # out of range: empty
    return idx


@pytest.mark.parametrize("tpg", [1, 2, 3, 4])
def test_union_is_the_set_union_in_first_occurrence_order(tpg):
    N = 500
    idx = _random_lists(12, 96, N, 0.6, 0.1, 40 + tpg)
    union, count = oracle.group_union_ref(idx, tpg, N, 400)
    for g in range(12 // tpg):
        lists = idx[g * tpg:(g + 1) * tpg]
        flat = lists.reshape(-1)
        ok = (flat >= 0) & (flat < N)
        vals = flat[ok]
        uniq, first = np.unique(vals, return_index=True)      # set union, first positions
        want = uniq[np.argsort(first)]                       # first-occurrence order
        assert count[g] == len(want)
        got = union[g, :count[g]].astype(np.int64)
        assert np.array_equal(got & oracle.grouping.ROW_MASK, want)
        for j, row in enumerate(want):                       # member bits = membership
            bits = [(row in set(lists[i][(lists[i] >= 0) & (lists[i] < N)].tolist())) for i in range(tpg)]
            assert (int(got[j]) >> oracle.grouping.MEMBER_SHIFT) == sum(1 << i for i, b in enumerate(bits) if b)
        assert np.all(union[g, count[g]:] == -1)


def test_union_overflow_keeps_the_first_entries():
    N = 300
    idx = _random_lists(4, 64, N, 0.0, 0.0, 7)
    full, cfull = oracle.group_union_ref(idx, 4, N, 256)
    cut, ccut = oracle.group_union_ref(idx, 4, N, 100)
    assert ccut[0] == cfull[0] > 100
    assert np.array_equal(cut[0], full[0, :100])


def test_grouped_decode_equals_per_token_decode():
    wl = W.custom(T=8, H=4, pool_rows=400, topk=48, empty_frac=0.0, seed=33)
    pool = oracle.nvfp4_pack_rows_ref(W.pool_source(wl))
    q = W.queries(wl)
    idx = _random_lists(8, 48, 400, 0.5, 0.15, 34)
    ref_idx = idx.copy()
    ref_idx[ref_idx >= 400] = -1
    want_o, want_l = oracle.sparse_mla_decode_ref(q, pool, ref_idx, wl.softmax_scale)
    for tpg in (1, 2, 4):
        union, count = oracle.group_union_ref(idx, tpg, 400, 4 * 48)
        got_o, got_l = oracle.sparse_mla_decode_grouped_ref(q, pool, union, tpg, wl.softmax_scale)
        # the same rows per token, only their order differs: equal up to summation order
        assert np.max(np.abs(got_o.astype(np.float64) - want_o)) <= 1e-3 * np.max(np.abs(want_o))
        assert np.allclose(got_l, want_l, rtol=0, atol=1e-9, equal_nan=False)

"""Pins of the oracle's top-k selection (the sparse indexer's list-producing step)
against a hand-worked example, the selection rule checked by brute force, and
torch.topk on distinct scores."""

import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "topk_example.json")


def _f(v):
    return float(v)


def test_topk_matches_hand_worked_example():
    ex = json.load(open(GOLDEN))
    scores = np.array([[_f(v) for v in row] for row in ex["scores"]], dtype=np.float32)
    got = oracle.topk_indices_ref(scores, ex["lengths"], ex["k"], ex["row_offset"])
    assert got.tolist() == ex["expected"]


def _brute(scores, lengths, k, off):
    """Position p of token t is chosen iff fewer than k positions beat it, where q beats
    p when its score is larger, or equal with q < p."""
    T, S = scores.shape
    out = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        n = int(lengths[t])
        s = [float(x) for x in scores[t, :n]]
        chosen = [p for p in range(n)
                  if sum(1 for q in range(n) if s[q] > s[p] or (s[q] == s[p] and q < p)) < k]
        out[t, :len(chosen)] = np.array(chosen) + off[t]
    return out


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force_with_many_ties(seed):
    rng = np.random.default_rng(seed)
    T, S = 5, 40
    scores = rng.integers(-3, 4, size=(T, S)).astype(np.float32)   # few distinct values: many ties
    scores[rng.random((T, S)) < 0.1] = -0.0
    scores[rng.random((T, S)) < 0.05] = -np.inf
    lengths = rng.integers(0, S + 1, size=T)
    off = rng.integers(0, 1000, size=T)
    for k in (1, 3, 17, 40, 55):
        assert np.array_equal(oracle.topk_indices_ref(scores, lengths, k, off), _brute(scores, lengths, k, off))


def test_topk_matches_torch_topk_on_distinct_scores():
    rng = np.random.default_rng(9)
    T, S, k = 3, 6000, 2048
    scores = rng.permutation(T * S).reshape(T, S).astype(np.float32) * 0.5 - 4000.0   # distinct, exact
    lengths = np.array([S, 4000, 2500])
    got = oracle.topk_indices_ref(scores, lengths, k)
    for t in range(T):
        n = lengths[t]
        ref = torch.topk(torch.from_numpy(scores[t, :n]), k).indices.numpy()
        assert np.array_equal(got[t], np.sort(ref))


def test_topk_output_is_sorted_unique_and_in_range():
    rng = np.random.default_rng(4)
    scores = rng.standard_normal((4, 3000)).astype(np.float32)
    lengths = np.array([3000, 2048, 100, 2049])
    got = oracle.topk_indices_ref(scores, lengths, 2048, [10, 20, 30, 40])
    for t, n in enumerate(lengths):
        v = got[t][got[t] >= 0]
        assert len(v) == min(2048, n)
        assert np.all(np.diff(v) > 0) and v.min() >= 10 * (t + 1) and v.max() < 10 * (t + 1) + n
        assert np.all(got[t][len(v):] == -1)


def test_topk_rejects_nan_and_bad_lengths():
    s = np.zeros((1, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.topk_indices_ref(np.full((1, 4), np.nan, dtype=np.float32), [4], 2)
    with pytest.raises(ValueError):
        oracle.topk_indices_ref(s, [5], 2)

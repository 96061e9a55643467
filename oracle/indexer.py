"""Top-k selection of the sparse indexer.  TEST INFRASTRUCTURE ONLY (see package doc).

"Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section
"Four-bit caches make room": the sparse indexer chooses, for each decode token, the
2,048 context positions whose cache rows the attention kernel loads.  The page gives
no internals of the indexer (its scores come from trained weights); what is stated
here is the selection step over given scores, the step that produces the index lists.

Readings taken where the page leaves the step open:
  * Token t has lengths[t] context positions 0 .. lengths[t] - 1 with float32 scores;
    its list holds the k positions with the largest scores.  Equal scores (compared
    as numbers, so -0 equals +0) go to the lower position.  Scores are not NaN.
  * The list is in ascending position order (a set has no order of its own; this one
    is unique and is the order a gather streams best in).
  * A token with fewer than k positions lists them all, then -1 (empty entries).
  * Entry = row_offset[t] + position: the pool row of the position (0 if no offsets).
"""

import numpy as np


def topk_indices_ref(scores, lengths, k, row_offset=None):
    """scores float32 [T, S], lengths int [T] (each <= S) -> int32 [T, k]."""
    scores = np.asarray(scores)
    if scores.dtype != np.float32 or scores.ndim != 2:
        raise ValueError("scores must be float32 [T, S]")
    T, S = scores.shape
    lengths = np.asarray(lengths, dtype=np.int64)
    if lengths.shape != (T,) or np.any(lengths < 0) or np.any(lengths > S):
        raise ValueError("lengths must be int [T] within [0, S]")
    if np.any(np.isnan(scores)):
        raise ValueError("scores must not be NaN")
    off = np.zeros(T, dtype=np.int64) if row_offset is None else np.asarray(row_offset, dtype=np.int64)
    out = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        n = int(lengths[t])
        s = scores[t, :n]
        # primary key: score, largest first; secondary: position, lowest first
        order = np.lexsort((np.arange(n), -s.astype(np.float64)))
        chosen = np.sort(order[:min(k, n)])
        out[t, :len(chosen)] = chosen + off[t]
    return out

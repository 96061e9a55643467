"""Grouped decode of token groups over union lists.  TEST INFRASTRUCTURE ONLY (see package doc).

"Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily": the decode tokens
of one agent session select largely the same cache rows, so the rows of a session can be
loaded once for all of its tokens.  The library's grouped decode does that in two steps;
these are their plain statements.

  * group_union_ref: for each group of `tpg` consecutive tokens, the rows that some token
    of the group lists (0 <= entry < pool_rows), once each, in order of first occurrence
    when the group's lists are read token by token from their first entry; every entry
    is row | members << 27, bit i of members set when token i of the group lists the row.
    The list is cut after U entries and padded with -1; the count is the full size.
  * sparse_mla_decode_grouped_ref: each token attends over the rows of its group's union
    whose member bit for that token is set -- by definition the same rows as its own list
    (lists without repeated rows), so the result is sparse_mla_decode_ref's.
"""

import numpy as np

from .attention import sparse_mla_decode_ref

MEMBER_SHIFT = 27
ROW_MASK = (1 << MEMBER_SHIFT) - 1


def group_union_ref(indices, tpg, pool_rows, U):
    """indices int32 [T, K] -> (union int32 [T // tpg, U], count int32 [T // tpg])."""
    indices = np.asarray(indices)
    T, K = indices.shape
    if T % tpg != 0:
        raise ValueError("T must be a multiple of tpg")
    G = T // tpg
    union = np.full((G, U), -1, dtype=np.int32)
    count = np.zeros(G, dtype=np.int32)
    for g in range(G):
        order = []          # rows in order of first occurrence
        members = {}        # row -> member bits
        for i in range(tpg):
            for v in indices[g * tpg + i]:
                v = int(v)
                if v < 0 or v >= pool_rows:
                    continue
                if v not in members:
                    members[v] = 0
                    order.append(v)
                members[v] |= 1 << i
        count[g] = len(order)
        for j, v in enumerate(order[:U]):
            union[g, j] = v | (members[v] << MEMBER_SHIFT)
    return union, count


def sparse_mla_decode_grouped_ref(q, pool, union, tpg, softmax_scale, tokens=None):
    """Grouped decode: q fp16 [T, H, 576], union int32 [T // tpg, U] -> (out, lse) as
    sparse_mla_decode_ref, each token over the union rows its member bit marks."""
    union = np.asarray(union)
    T = q.shape[0]
    lists = np.full((T, union.shape[1]), -1, dtype=np.int64)
    for t in range(T):
        g, i = divmod(t, tpg)
        e = union[g].astype(np.int64)
        sel = (e >= 0) & (((e >> MEMBER_SHIFT) >> i) & 1 == 1)
        rows = e[sel] & ROW_MASK
        lists[t, :len(rows)] = rows
    return sparse_mla_decode_ref(q, pool, lists, softmax_scale, tokens=tokens)

"""GPU parity of the 64-head decode on lists that end in runs of empty entries, through
the C ABI, against the oracle.

A token whose context is shorter than the list length ends its list in a run of empty
entries ("Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily", section
"Four-bit caches make room": the kernel handles empty list entries).  The lists here mix
every length that matters to the tiles of 64 entries -- no row at all, one row, a tile
boundary just missed, hit and passed, the whole list -- with out-of-pool entries at the
end (empty as well), whole empty tiles inside a list and scattered empties, at split
counts from one range per launch to several per token, 64 and 128 heads, and a list length
that is not a multiple of the tile.
"""

import sys

import numpy as np
import pytest

import oracle
from sparse_mla_decode_04_amd import workloads as W
from helpers import OracleRows, assert_parity, build_device_pool

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def smla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_decode_04_amd as m
    m.lib()
    return m


def _np(t):
    return t.detach().cpu().numpy()


def trailing_empty_lists(T, K, N, seed):
    """int32 [T, K] lists of distinct pool rows with per-token valid prefixes of the lengths
    that matter to the cut, out-of-pool entries past some prefixes, an empty tile inside some
    lists and scattered empties in others."""
    rng = np.random.default_rng(seed)
    special = [0, 1, 63, 64, 65, 128, K - 1, K, 2 * 64 + 1]
    idx = np.full((T, K), -1, dtype=np.int64)
    for t in range(T):
        n = special[t] if t < len(special) else int(rng.integers(0, K + 1))
        n = min(n, K)
        idx[t, :n] = rng.choice(N, size=n, replace=False) if n <= N else rng.integers(0, N, size=n)
        if t % 3 == 1 and n < K:          # past the prefix: rows beyond the pool (empty as well)
            m = int(rng.integers(1, K - n + 1))
            idx[t, n:n + m] = N + rng.integers(0, 1000, size=m)
        if t % 4 == 2 and n >= 3 * 64:    # a whole empty tile inside the list
            idx[t, 64:128] = -1
        if t % 5 == 3 and n > 0:          # scattered empties inside the prefix
            idx[t, rng.choice(n, size=max(1, n // 7), replace=False)] = -1
    return idx.astype(np.int32)


CASES = [  # T, H, N, K, seed, num_splits
    (12, 64, 6000, 2048, 1, 0),      # several ranges per token, each inside one token
    (12, 64, 6000, 2048, 2, 30),     # ranges across token boundaries
    (12, 64, 6000, 2048, 3, 20),
    (12, 64, 6000, 2048, 4, 7),
    (12, 64, 6000, 2048, 5, 1),      # one range over every tile
    (20, 64, 3000, 2048, 6, 1),
    (40, 128, 5000, 2048, 7, 0),     # two head blocks
    (40, 128, 5000, 2048, 8, 50),
    (9, 64, 3000, 700, 9, 0),        # a ragged last tile
    (9, 64, 3000, 700, 10, 5),
    (300, 64, 5000, 512, 11, 0),     # more tokens than ranges
]


@pytest.mark.parametrize("T,H,N,K,seed,splits", CASES)
def test_trailing_empties_match_oracle(smla, T, H, N, K, seed, splits):
    _say("trailing empties", T, H, N, K, seed, splits)
    wl = W.custom(T=T, H=H, pool_rows=N, topk=K, seed=100 + seed)
    src = W.pool_source(wl)
    q = W.queries(wl)
    idx = trailing_empty_lists(T, K, N, seed)
    pool = build_device_pool(src, DEV)
    out, lse = smla.sparse_mla_decode(torch.from_numpy(q).to(DEV), pool, torch.from_numpy(idx).to(DEV),
                                      wl.softmax_scale, num_splits=splits)
    toks = list(range(T)) if T <= 40 else sorted(set(list(range(12)) + list(range(12, T, 7)) + [T - 1]))
    # the boundary reads an entry at or past the pool's end as empty: the oracle gets -1 there
    ref_idx = np.where(idx < N, idx, -1).astype(np.int32)
    ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src), ref_idx, wl.softmax_scale, tokens=toks)
    assert_parity(_np(out)[toks], _np(lse)[toks], ref_o, ref_l, f"trailing empties T={T} H={H} K={K} splits={splits}")
    empty = np.nonzero(~np.any((idx >= 0) & (idx < N), axis=1))[0]
    assert np.all(_np(out)[empty] == 0) and np.all(np.isneginf(_np(lse)[empty]))


def test_workspace_reuse_with_new_lists(smla):
    """One workspace, three calls whose lists end at different places (the merge counters
    are left at zero for the next call)."""
    T, H, N, K = 10, 64, 4000, 2048
    wl = W.custom(T=T, H=H, pool_rows=N, topk=K, seed=140)
    src = W.pool_source(wl)
    q = W.queries(wl)
    pool = build_device_pool(src, DEV)
    ws = smla.make_workspace(T, H, K, 0, DEV)
    qd = torch.from_numpy(q).to(DEV)
    for seed in (21, 22, 23):
        idx = trailing_empty_lists(T, K, N, seed)
        rng = np.random.default_rng(seed)
        rng.shuffle(idx)   # the special lengths land on other tokens each call
        out, lse = smla.sparse_mla_decode(qd, pool, torch.from_numpy(idx).to(DEV), wl.softmax_scale, workspace=ws)
        ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src), np.where(idx < N, idx, -1).astype(np.int32),
                                                    wl.softmax_scale)
        assert_parity(_np(out), _np(lse), ref_o, ref_l, f"reuse seed {seed}")

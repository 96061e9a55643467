"""GPU parity of grouped decode (called through the C ABI) against the CPU oracle.

Bit-exact: the union lists of token groups (smla_group_union) against
oracle.group_union_ref.  Within tolerance (max |out - ref| <= 2e-3 max |ref|,
|lse - ref| <= 1e-3, -inf exactly where the oracle has it):
sparse_mla_decode_grouped on those lists against the per-token oracle decode
of the tokens' own lists, for groups of 4 x 16, 2 x 32 and 1 x 64 heads, ragged
list lengths, empty entries, empty tokens and every kind of split.
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


def session_lists(T, K, N, tpg, shared, empty_frac, seed):
    """T lists of K distinct rows from [0, N); each group of tpg tokens shares a fraction
    `shared` of its rows (the rest of each list is the token's own); some entries empty
    (-1) or out of range (>= N)."""
    rng = np.random.default_rng(seed)
    idx = np.empty((T, K), dtype=np.int32)
    for g in range(0, T, tpg):
        perm = rng.permutation(N)
        ns = int(shared * K)
        common, pos = perm[:ns], ns
        for t in range(g, g + tpg):
            own = perm[pos:pos + K - ns]
            pos += K - ns
            idx[t] = rng.permutation(np.concatenate([common, own]))
    idx[rng.random(idx.shape) < empty_frac] = -1
    idx[rng.random(idx.shape) < 0.01] = N + 5
    return idx


@pytest.mark.parametrize("tpg,K,U", [(1, 300, 300), (2, 700, 1400), (3, 200, 600), (4, 2048, 8192),
                                     (4, 512, 800)])
def test_union_bit_exact(smla, tpg, K, U):
    _say("union", tpg, K, U)
    N = 20000
    idx = session_lists(4 * tpg, K, N, tpg, 0.75, 0.05, 50 + tpg)
    uni, cnt = smla.group_union(torch.from_numpy(idx).to(DEV), tpg, N, U)
    ref_u, ref_c = oracle.group_union_ref(idx, tpg, N, U)
    assert np.array_equal(_np(cnt), ref_c)
    assert np.array_equal(_np(uni), ref_u)


def _grouped_case(T, H, tpg, N, K, shared, empty_frac, seed):
    wl = W.custom(T=T, H=H, pool_rows=N, topk=K, empty_frac=0.0, seed=seed)
    src = W.pool_source(wl)
    q = W.queries(wl)
    idx = session_lists(T, K, N, tpg, shared, empty_frac, seed + 1)
    ref_idx = idx.copy()
    ref_idx[ref_idx >= N] = -1
    return wl, src, q, idx, ref_idx


@pytest.mark.parametrize("T,H,tpg,K,splits", [
    (8, 16, 4, 700, 0),      # ragged union length
    (8, 16, 4, 2048, 0),
    (8, 16, 4, 2048, 1),
    (8, 16, 4, 2048, 7),
    (8, 16, 4, 2048, 1000),  # one tile per workgroup
    (6, 32, 2, 1000, 0),
    (3, 64, 1, 900, 3),
])
def test_grouped_decode_matches_per_token_oracle(smla, T, H, tpg, K, splits):
    _say("grouped decode", T, H, tpg, K, splits)
    N = 30000
    wl, src, q, idx, ref_idx = _grouped_case(T, H, tpg, N, K, 0.75, 0.05, 60 + K + splits)
    pool = build_device_pool(src, DEV)
    U = tpg * K
    uni, cnt = smla.group_union(torch.from_numpy(idx).to(DEV), tpg, N, U)
    out, lse = smla.sparse_mla_decode_grouped(torch.from_numpy(q).to(DEV), pool, uni, tpg, wl.softmax_scale,
                                              num_splits=splits)
    ref_out, ref_lse = oracle.sparse_mla_decode_ref(q, OracleRows(src), ref_idx, wl.softmax_scale)
    assert_parity(_np(out), _np(lse), ref_out, ref_lse, f"grouped T{T} H{H} tpg{tpg} K{K} splits{splits}")


def test_grouped_empty_tokens_and_unshared_groups(smla):
    N = 8000
    wl, src, q, idx, ref_idx = _grouped_case(8, 16, 4, N, 256, 0.0, 0.0, 71)   # nothing shared
    idx[1, :] = -1                      # a token with an empty list
    idx[4:8, :] = -1                    # a whole group empty
    ref_idx = idx.copy()
    ref_idx[ref_idx >= N] = -1
    pool = build_device_pool(src, DEV)
    uni, cnt = smla.group_union(torch.from_numpy(idx).to(DEV), 4, N, 1024)
    assert _np(cnt)[1] == 0
    out, lse = smla.sparse_mla_decode_grouped(torch.from_numpy(q).to(DEV), pool, uni, 4, wl.softmax_scale)
    ref_out, ref_lse = oracle.sparse_mla_decode_ref(q, OracleRows(src), ref_idx, wl.softmax_scale)
    assert_parity(_np(out), _np(lse), ref_out, ref_lse, "grouped empties")
    assert np.all(_np(out)[[1, 4, 5, 6, 7]] == 0) and np.all(np.isneginf(_np(lse)[[1, 4, 5, 6, 7]]))


def test_grouped_decode_is_deterministic(smla):
    N = 20000
    wl, src, q, idx, _ = _grouped_case(8, 16, 4, N, 2048, 0.75, 0.02, 81)
    pool = build_device_pool(src, DEV)
    idx_d, q_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(q).to(DEV)
    a = smla.sparse_mla_decode_grouped(q_d, pool, smla.group_union(idx_d, 4, N, 8192)[0], 4, wl.softmax_scale)
    b = smla.sparse_mla_decode_grouped(q_d, pool, smla.group_union(idx_d, 4, N, 8192)[0], 4, wl.softmax_scale)
    assert np.array_equal(_np(a[0]).view(np.uint16), _np(b[0]).view(np.uint16))
    assert np.array_equal(_np(a[1]), _np(b[1]))

"""Pins of the oracle's sparse MLA decode, LSE combine and staged variant against
torch's scaled_dot_product_attention / logsumexp in float64, closed forms and
invariants (permutation, added empties, identical rows, single entry, split
then combine)."""

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_decode_04_amd import workloads as W


def _case(T=3, H=4, N=64, K=16, empty_frac=0.25, seed=21):
    wl = W.custom(T=T, H=H, pool_rows=N, topk=K, empty_frac=empty_frac, seed=seed)
    pool = oracle.nvfp4_pack_rows_ref(W.pool_source(wl))
    return wl, W.queries(wl), pool, W.index_lists(wl)


def _decode64(q, pool, idx, scale):
    """fp64 output (before the final fp16 rounding) via the oracle's internals."""
    from oracle.attention import _attend
    outs, lses = [], []
    for t in range(q.shape[0]):
        ids = idx[t][idx[t] >= 0]
        K = oracle.dense_rows_for(pool, ids) if len(ids) else np.zeros((0, 576))
        o, l = _attend(q[t].astype(np.float64), K, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def test_matches_torch_sdpa_and_logsumexp_fp64():
    wl, q, pool, idx = _case()
    out, lse = oracle.sparse_mla_decode_ref(q, pool, idx, wl.softmax_scale)
    for t in range(wl.T):
        ids = idx[t][idx[t] >= 0]
        K = torch.from_numpy(oracle.nvfp4_unpack_rows_ref(pool[ids]))           # [n, 576]
        Q = torch.from_numpy(q[t].astype(np.float64))                          # [H, 576]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None, :, None, :], K[None, None].expand(1, wl.H, -1, -1),
            K[None, None, :, :512].expand(1, wl.H, -1, -1), scale=wl.softmax_scale)[0, :, 0]
        ref16 = ref.numpy().astype(np.float16)
        assert np.array_equal(out[t].view(np.uint16), ref16.view(np.uint16)) or \
            np.max(np.abs(out[t].astype(np.float64) - ref.numpy())) <= 1e-3 * np.max(np.abs(ref.numpy())) * 2 ** -9
        lref = torch.logsumexp((Q @ K.T) * wl.softmax_scale, dim=1).numpy()
        assert np.allclose(lse[t], lref, rtol=0, atol=1e-12)


def test_sdpa_catches_transposed_or_partial_use_of_the_row():
    # the rope half must enter the scores and must not enter the output
    wl, q, pool, idx = _case(T=1, H=2, K=8, empty_frac=0.0)
    o64, l64 = _decode64(q, pool, idx, wl.softmax_scale)
    K = oracle.nvfp4_unpack_rows_ref(pool[idx[0]])
    s = (K @ q[0].astype(np.float64).T) * wl.softmax_scale
    s_lat = (K[:, :512] @ q[0, :, :512].astype(np.float64).T) * wl.softmax_scale
    assert not np.allclose(s, s_lat)
    l_ref = torch.logsumexp(torch.from_numpy(s), dim=0).numpy()
    assert np.allclose(l64[0], l_ref, atol=1e-12)


def test_index_permutation_invariance():
    wl, q, pool, idx = _case(T=2, K=32)
    rng = np.random.default_rng(1)
    perm = np.stack([rng.permutation(idx.shape[1]) for _ in range(idx.shape[0])])
    idx2 = np.take_along_axis(idx, perm, axis=1)
    o1, l1 = _decode64(q, pool, idx, wl.softmax_scale)
    o2, l2 = _decode64(q, pool, idx2, wl.softmax_scale)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-15)
    assert np.allclose(l1, l2, rtol=0, atol=1e-13)


def test_adding_empty_entries_changes_nothing():
    wl, q, pool, idx = _case(T=2, K=24, empty_frac=0.0)
    padded = np.full((idx.shape[0], 64), -1, dtype=np.int32)
    rng = np.random.default_rng(2)
    for t in range(idx.shape[0]):
        pos = np.sort(rng.choice(64, size=idx.shape[1], replace=False))
        padded[t, pos] = idx[t]
    o1, l1 = oracle.sparse_mla_decode_ref(q, pool, idx, wl.softmax_scale)
    o2, l2 = oracle.sparse_mla_decode_ref(q, pool, padded, wl.softmax_scale)
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16))
    assert np.array_equal(l1, l2)


def test_identical_rows_give_the_latent_exactly_and_lse_plus_log_n():
    wl, q, pool, _ = _case(T=1, H=3, N=8, K=8)
    for n in (1, 2, 5, 37):
        idx = np.full((1, 40), -1, dtype=np.int32)
        idx[0, :n] = 3                      # the same row n times (counted per entry)
        out, lse = oracle.sparse_mla_decode_ref(q, pool, idx, wl.softmax_scale)
        K = oracle.nvfp4_unpack_rows_ref(pool[3:4])[0]
        v16 = K[:512].astype(np.float16)
        for h in range(wl.H):
            # value equality: a sum of weighted -0 entries is +0, the sign of zero carries nothing
            assert np.array_equal(out[0, h], v16)
            s = wl.softmax_scale * float(np.dot(q[0, h].astype(np.float64), K))
            assert abs(lse[0, h] - (s + math.log(n))) < 1e-12


def test_single_entry_gives_that_row():
    wl, q, pool, _ = _case(T=1, H=2, N=16, K=8)
    idx = np.full((1, 8), -1, dtype=np.int32)
    idx[0, 5] = 11
    out, lse = oracle.sparse_mla_decode_ref(q, pool, idx, wl.softmax_scale)
    K = oracle.nvfp4_unpack_rows_ref(pool[11:12])[0]
    for h in range(2):
        assert np.array_equal(out[0, h], K[:512].astype(np.float16))
        assert abs(lse[0, h] - wl.softmax_scale * float(np.dot(q[0, h].astype(np.float64), K))) < 1e-12


def test_all_empty_list_gives_zero_and_minus_inf():
    wl, q, pool, idx = _case(T=2, K=8)
    idx[1, :] = -1
    out, lse = oracle.sparse_mla_decode_ref(q, pool, idx, wl.softmax_scale)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(lse[0]))


def test_two_row_hand_example():
    # row 0 latent all 6 (amax 6 -> scale exactly 1, code 7), row 1 latent all 3 (amax 3 ->
    # scale exactly 0.5, code 6), rope zero; one head with q = 2^-9 on the latent: the dot
    # products are 6 and 3, scores s = 0.5*6 and 0.5*3; closed-form two-term softmax.
    src = np.zeros((2, 576), dtype=np.float16)
    src[0, :512] = 6.0
    src[1, :512] = 3.0
    pool = oracle.nvfp4_pack_rows_ref(src)
    q = np.zeros((1, 1, 576), dtype=np.float16)
    q[0, 0, :512] = 1.0 / 512          # exact in fp16 (2^-9)
    scale = 0.5
    out, lse = oracle.sparse_mla_decode_ref(q, pool, np.array([[0, -1, 1]], dtype=np.int32), scale)
    s1, s2 = 3.0, 1.5
    l_exp = math.log(math.exp(s1) + math.exp(s2))
    w1 = math.exp(s1 - l_exp)
    o_exp = w1 * 6.0 + (1 - w1) * 3.0
    assert abs(lse[0, 0] - l_exp) < 1e-14
    assert np.all(out[0, 0] == np.float16(o_exp))


def test_split_then_combine_equals_unsplit():
    wl, q, pool, idx = _case(T=3, H=4, N=200, K=96, empty_frac=0.3)
    o_all, l_all = _decode64(q, pool, idx, wl.softmax_scale)
    for S in (1, 2, 3, 7):
        bounds = np.linspace(0, idx.shape[1], S + 1).astype(int)
        po, pl = [], []
        for s in range(S):
            sub = np.full_like(idx, -1)
            sub[:, bounds[s]:bounds[s + 1]] = idx[:, bounds[s]:bounds[s + 1]]
            o, l = _decode64(q, pool, sub, wl.softmax_scale)
            po.append(o)
            pl.append(l)
        out, lse = oracle.lse_combine_ref(np.stack(po), np.stack(pl))
        assert np.allclose(out, o_all, rtol=1e-12, atol=1e-14)
        assert np.allclose(lse, l_all, rtol=0, atol=1e-12)


def test_combine_ignores_minus_inf_partials_and_all_empty():
    po = np.array([[[1.0, 2.0]], [[5.0, 7.0]], [[9.0, 9.0]]])
    pl = np.array([[0.3], [-np.inf], [-np.inf]])
    out, lse = oracle.lse_combine_ref(po, pl)
    assert np.allclose(out, [[1.0, 2.0]]) and np.allclose(lse, [0.3])
    out, lse = oracle.lse_combine_ref(po, np.full((3, 1), -np.inf))
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    # equal lse halves: plain mean, lse + ln 2
    out, lse = oracle.lse_combine_ref(po[:2], np.array([[1.0], [1.0]]))
    assert np.allclose(out, [[3.0, 4.5]]) and np.allclose(lse, [1.0 + math.log(2)])


def test_staged_equals_fused_when_fp8_is_exact():
    # scales that are powers of two and E2M1 values make every product E4M3-exact
    rng = np.random.default_rng(4)
    src = np.zeros((6, 576), dtype=np.float16)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    for i in range(6):
        pw = 2.0 ** rng.integers(-3, 3, size=32)
        vals = rng.choice(grid, size=(32, 16)) * rng.choice([-1, 1], size=(32, 16))
        vals[:, 0] = 6.0                       # amax 6*pw -> scale exactly pw
        src[i, :512] = (vals * pw[:, None]).reshape(-1)
        src[i, 512:] = rng.choice(grid, size=64)
    pool = oracle.nvfp4_pack_rows_ref(src)
    q = rng.standard_normal((2, 3, 576)).astype(np.float16)
    idx = np.array([[0, 1, 2, -1, 3], [5, -1, 4, 2, 0]], dtype=np.int32)
    o1, l1 = oracle.sparse_mla_decode_ref(q, pool, idx, 1 / 24)
    o2, l2 = oracle.sparse_mla_decode_fp8rows_ref(q, pool, idx, 1 / 24)
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16)) and np.array_equal(l1, l2)


def test_staged_differs_from_fused_on_gaussian_rows():
    wl, q, pool, idx = _case(T=2, H=4, N=64, K=32, empty_frac=0.0)
    o1, _ = oracle.sparse_mla_decode_ref(q, pool, idx, wl.softmax_scale)
    o2, _ = oracle.sparse_mla_decode_fp8rows_ref(q, pool, idx, wl.softmax_scale)
    assert not np.array_equal(o1, o2)


def test_rejects_bad_shapes():
    wl, q, pool, idx = _case(T=1, K=8)
    with pytest.raises(ValueError):
        oracle.sparse_mla_decode_ref(q.astype(np.float32), pool, idx, 0.1)
    with pytest.raises(ValueError):
        oracle.sparse_mla_decode_ref(q, pool, idx[0], 0.1)

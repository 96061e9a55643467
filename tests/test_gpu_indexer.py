"""GPU parity of the sparse indexer's top-k selection (sparse_indexer_topk, called
through the C ABI) against oracle.topk_indices_ref, bit for bit: ties at the cut (-0
and +0 equal), infinities, subnormals, all-equal scores, lengths of 0, below, at and
above k with ragged tails, with and without row offsets; the full-size synthetic
inputs of the 35- and 264-token workloads; and the lists it produces driving
sparse_mla_decode."""

import sys

import numpy as np
import pytest

import oracle
from sparse_mla_decode_04_amd import workloads as W
from helpers import OracleRows, assert_parity, build_device_pool, pool_source_all

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


def _scores(kind, T, S, rng):
    if kind == "normal":
        return rng.standard_normal((T, S)).astype(np.float32)
    if kind == "ties":
        return rng.integers(-4, 5, size=(T, S)).astype(np.float32)
    if kind == "grid":
        return (np.round(rng.standard_normal((T, S)) * 64) / 64).astype(np.float32)
    if kind == "specials":
        s = rng.standard_normal((T, S)).astype(np.float32)
        r = rng.random((T, S))
        s[r < 0.2] = -0.0
        s[(r >= 0.2) & (r < 0.35)] = 0.0
        s[(r >= 0.35) & (r < 0.4)] = -np.inf
        s[(r >= 0.4) & (r < 0.42)] = np.inf
        s[(r >= 0.42) & (r < 0.5)] = np.float32(1e-40) * rng.integers(-5, 6, size=int(np.sum((r >= 0.42) & (r < 0.5))))
        return s
    if kind == "equal":
        return np.full((T, S), 0.25, dtype=np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "ties", "grid", "specials", "equal"])
@pytest.mark.parametrize("k", [1, 7, 300, 2048])
def test_topk_bit_exact(smla, kind, k):
    _say("topk", kind, k)
    rng = np.random.default_rng(["normal", "ties", "grid", "specials", "equal"].index(kind) * 100000 + k)
    T, S = 9, 5000
    scores = _scores(kind, T, S, rng)
    lengths = np.array([S, 0, k - 1 if k > 1 else 0, k, k + 1, 4999, 4097, 1234, S], dtype=np.int32)
    off = rng.integers(0, 100000, size=T).astype(np.int32)
    for use_len, use_off in ((True, True), (True, False), (False, True)):
        got = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), k,
                                       torch.from_numpy(lengths).to(DEV) if use_len else None,
                                       torch.from_numpy(off).to(DEV) if use_off else None)
        ref = oracle.topk_indices_ref(scores, lengths if use_len else np.full(T, S), k, off if use_off else None)
        assert np.array_equal(got.cpu().numpy(), ref), (use_len, use_off)


def test_topk_large_k_and_long_rows(smla):
    rng = np.random.default_rng(12)
    T, S = 3, 200000
    scores = (np.round(rng.standard_normal((T, S)) * 16) / 16).astype(np.float32)
    lengths = np.array([S, 150001, 65537], dtype=np.int32)
    for k in (65536, 4096):
        got = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), k, torch.from_numpy(lengths).to(DEV))
        assert np.array_equal(got.cpu().numpy(), oracle.topk_indices_ref(scores, lengths, k))


@pytest.mark.parametrize("cfg", [2, 4])
def test_topk_full_size_workload(smla, cfg):
    wl = W.WORKLOADS[cfg]
    _say(f"topk config {cfg} {wl.name}")
    scores, lengths, off = W.indexer_inputs(wl)
    got = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), wl.topk, torch.from_numpy(lengths).to(DEV),
                                   torch.from_numpy(off).to(DEV)).cpu().numpy()
    ref = oracle.topk_indices_ref(scores, lengths, wl.topk, off)
    bad = np.nonzero(np.any(got != ref, axis=1))[0]
    assert bad.size == 0, f"{bad.size} tokens differ, first {bad[:5].tolist()}"


def test_indexer_lists_drive_decode(smla):
    """The selection's lists feed the decode kernel directly (35-token workload)."""
    wl = W.WORKLOADS[2]
    scores, lengths, off = W.indexer_inputs(wl)
    src = pool_source_all(wl)
    pool = build_device_pool(src, DEV)
    q = W.queries(wl)
    idx_d = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), wl.topk, torch.from_numpy(lengths).to(DEV),
                                     torch.from_numpy(off).to(DEV))
    out, lse = smla.sparse_mla_decode(torch.from_numpy(q).to(DEV), pool, idx_d, wl.softmax_scale)
    ref_idx = oracle.topk_indices_ref(scores, lengths, wl.topk, off)
    toks = [0, 11, 34]
    ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src), ref_idx, wl.softmax_scale, tokens=toks)
    assert_parity(out.cpu().numpy()[toks], lse.cpu().numpy()[toks], ref_o, ref_l, "indexer -> decode")


@pytest.mark.parametrize("kind", ["equal", "grid"])
def test_topk_crowded_cut_bin(smla, kind):
    """Far more keys share the cut's top 11 bits than LDS keeps (all equal, or three
    values): the selection finishes from the scores in memory."""
    rng = np.random.default_rng(21)
    T, S = 4, 60000
    scores = _scores(kind, T, S, rng) if kind == "equal" else rng.integers(0, 3, size=(T, S)).astype(np.float32)
    lengths = np.array([S, 50001, 40000, 2049], dtype=np.int32)
    for k in (2048, 100):
        got = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), k, torch.from_numpy(lengths).to(DEV))
        assert np.array_equal(got.cpu().numpy(), oracle.topk_indices_ref(scores, lengths, k))


def test_topk_context_longer_than_the_bitmaps(smla):
    """Contexts of more than 147,456 positions take the path that reads the scores again."""
    rng = np.random.default_rng(31)
    T, S = 4, 300000
    scores = (np.round(rng.standard_normal((T, S)) * 64) / 64).astype(np.float32)
    lengths = np.array([S, 147457, 147456, 147455], dtype=np.int32)
    off = np.array([5, 0, 1000000, 7], dtype=np.int32)
    got = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), 2048, torch.from_numpy(lengths).to(DEV),
                                   torch.from_numpy(off).to(DEV))
    assert np.array_equal(got.cpu().numpy(), oracle.topk_indices_ref(scores, lengths, 2048, off))


# More tokens than compute units: the 512-thread workgroup form of the selection (smaller
# per-wave cut-bin buffers, other bin and scan widths) runs instead of the 1,024-thread one.
MANY_T = 300


@pytest.mark.parametrize("kind", ["ties", "grid", "specials", "equal"])
def test_topk_many_tokens_bit_exact(smla, kind):
    _say("topk many tokens", kind)
    rng = np.random.default_rng(["ties", "grid", "specials", "equal"].index(kind) + 700)
    S = 3000
    scores = _scores(kind, MANY_T, S, rng)
    lengths = rng.integers(0, S + 1, size=MANY_T).astype(np.int32)
    lengths[:4] = [0, 2047, 2048, 2049]
    off = rng.integers(0, 100000, size=MANY_T).astype(np.int32)
    for k in (2048, 300):
        got = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), k, torch.from_numpy(lengths).to(DEV),
                                       torch.from_numpy(off).to(DEV))
        assert np.array_equal(got.cpu().numpy(), oracle.topk_indices_ref(scores, lengths, k, off)), k


@pytest.mark.parametrize("kind", ["equal", "three"])
def test_topk_many_tokens_crowded_cut_bin(smla, kind):
    rng = np.random.default_rng(41)
    S = 20000
    scores = (np.full((MANY_T, S), 0.25, dtype=np.float32) if kind == "equal"
              else rng.integers(0, 3, size=(MANY_T, S)).astype(np.float32))
    lengths = rng.integers(2049, S + 1, size=MANY_T).astype(np.int32)
    for k in (2048, 100):
        got = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), k, torch.from_numpy(lengths).to(DEV))
        assert np.array_equal(got.cpu().numpy(), oracle.topk_indices_ref(scores, lengths, k)), k


def test_topk_many_tokens_long_context(smla):
    rng = np.random.default_rng(42)
    S = 150000
    scores = (np.round(rng.standard_normal((MANY_T, S)) * 64) / 64).astype(np.float32)
    lengths = rng.integers(140000, S + 1, size=MANY_T).astype(np.int32)
    lengths[:3] = [S, 147457, 147456]
    got = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), 2048, torch.from_numpy(lengths).to(DEV))
    assert np.array_equal(got.cpu().numpy(), oracle.topk_indices_ref(scores, lengths, 2048))


# Split selection: each token's positions over `parts` workgroups (histogram, classify and
# finish launches), bit-exact against the same oracle, with chunk boundaries, empty chunks
# (more workgroups than 32-position chunks), crowded cut bins (the finish from memory) and
# contexts longer than the bitmaps.
@pytest.mark.parametrize("kind", ["normal", "ties", "grid", "specials", "equal"])
@pytest.mark.parametrize("parts", [2, 3, 7, 64])
def test_topk_split_bit_exact(smla, kind, parts):
    _say("topk split", kind, parts)
    rng = np.random.default_rng(["normal", "ties", "grid", "specials", "equal"].index(kind) * 1000 + parts + 900)
    T, S = 7, 20000
    scores = _scores(kind, T, S, rng)
    lengths = np.array([S, 0, 2047, 2049, 2048 + 33, 19999, 4096 + 64 * 31], dtype=np.int32)
    off = rng.integers(0, 100000, size=T).astype(np.int32)
    for k in (2048, 300, 1):
        got = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), k, torch.from_numpy(lengths).to(DEV),
                                       torch.from_numpy(off).to(DEV), parts=parts)
        ref = oracle.topk_indices_ref(scores, lengths, k, off)
        assert np.array_equal(got.cpu().numpy(), ref), k


@pytest.mark.parametrize("kind", ["equal", "three"])
def test_topk_split_crowded_cut_bin(smla, kind):
    rng = np.random.default_rng(51)
    T, S = 3, 60000
    scores = (np.full((T, S), 0.25, dtype=np.float32) if kind == "equal"
              else rng.integers(0, 3, size=(T, S)).astype(np.float32))
    lengths = np.array([S, 50001, 2049], dtype=np.int32)
    for parts in (2, 9):
        got = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), 2048, torch.from_numpy(lengths).to(DEV),
                                       parts=parts)
        assert np.array_equal(got.cpu().numpy(), oracle.topk_indices_ref(scores, lengths, 2048)), parts


def test_topk_split_context_longer_than_the_bitmaps(smla):
    rng = np.random.default_rng(52)
    T, S = 3, 300000
    scores = (np.round(rng.standard_normal((T, S)) * 64) / 64).astype(np.float32)
    lengths = np.array([S, 147457, 147456], dtype=np.int32)
    got = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), 2048, torch.from_numpy(lengths).to(DEV),
                                   parts=16)
    assert np.array_equal(got.cpu().numpy(), oracle.topk_indices_ref(scores, lengths, 2048))


def test_topk_split_workspace_reuse(smla):
    """One workspace, calls with other scores, lengths and k: the counters the split keeps in
    it are left at zero for the next call."""
    rng = np.random.default_rng(53)
    T, S = 5, 40000
    ws = smla.make_indexer_workspace(T, S, 2048, 5, DEV)
    assert ws is not None
    for i, kind in enumerate(["grid", "ties", "specials", "equal"]):
        scores = _scores(kind, T, S, rng)
        lengths = rng.integers(0, S + 1, size=T).astype(np.int32)
        k = [2048, 700, 2048, 5][i]
        got = smla.sparse_indexer_topk(torch.from_numpy(scores).to(DEV), k, torch.from_numpy(lengths).to(DEV),
                                       parts=5, workspace=ws)
        assert np.array_equal(got.cpu().numpy(), oracle.topk_indices_ref(scores, lengths, k)), kind


def test_topk_automatic_split_is_used_for_few_tokens(smla):
    """The 35-token workload's shape gets a workspace (a split) by default; the 264-token one
    runs one workgroup per token."""
    assert smla.indexer_workspace_bytes(35, 140000, 2048) > 0
    assert smla.indexer_workspace_bytes(264, 146000, 2048) == 0

"""GPU parity of the HIP path (called through the C ABI) against the CPU oracle.

Bit-exact: the cache-row writer (nvfp4_pack_rows), the on-chip unpack
(nvfp4_unpack_rows_f16) and the staged FP8 re-encode (nvfp4_stage_fp8).
Within tolerance (max |out - ref| <= 2e-3 max |ref|, |lse - ref| <= 1e-3, -inf
exactly where the oracle has it): sparse_mla_decode, sparse_mla_combine and the
staged pass 2, on small shapes spanning several chunks and ragged tails, every
split count, the invariants of the method, and poisoned memory.
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
    m.lib()  # raises if the library is missing
    return m


def _np(t):
    return t.detach().cpu().numpy()


# ----------------------------------------------------------------------------- codec

def _edge_rows(rng, n):
    src = (rng.standard_normal((n, 576)) * rng.choice([1e-6, 1e-3, 0.1, 1, 7, 300, 3e4], size=(n, 1)))
    src = np.clip(src, -65504, 65504).astype(np.float16)    # finite inputs only
    src[0] = 0
    src[1] = -0.0
    src[2, :16] = np.float16(6.0)                 # amax 6 -> scale 1
    src[2, 16:32] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5, -6]
    src[3, :] = np.float16(65504)                  # saturating scales and rope
    src[4, ::2] = np.float16(-60000)
    src[5, :] = np.float16(6e-8)                   # fp16 subnormal amax -> zero scale
    return src


def test_pack_bit_exact(smla):
    rng = np.random.default_rng(101)
    n = 777
    src = _edge_rows(rng, n)
    _say("pack: n", n)
    N = 1000
    slots = rng.choice(N, size=n, replace=False).astype(np.int32)
    slots[7] = -1        # skipped
    slots[9] = N + 5     # out of range: skipped
    pool = torch.full((N, 352), 0xA5, dtype=torch.uint8, device=DEV)
    smla.nvfp4_pack_rows(torch.from_numpy(src).to(DEV), torch.from_numpy(slots).to(DEV), pool)
    got = _np(pool)
    ref = oracle.nvfp4_pack_rows_ref(src)
    ok = (slots >= 0) & (slots < N)
    bad = np.nonzero(np.any(got[slots[ok]] != ref[ok], axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first src row {np.nonzero(ok)[0][bad[0]]}"
    untouched = np.setdiff1d(np.arange(N), slots[ok])
    assert np.all(got[untouched] == 0xA5)


def test_pack_empty_batch_is_noop(smla):
    pool = torch.full((4, 352), 7, dtype=torch.uint8, device=DEV)
    smla.nvfp4_pack_rows(torch.zeros((0, 576), dtype=torch.float16, device=DEV),
                         torch.zeros((0,), dtype=torch.int32, device=DEV), pool)
    torch.cuda.synchronize()
    assert torch.all(pool == 7)


def _same_f16(a, b):
    a = np.asarray(a, dtype=np.float16)
    b = np.asarray(b, dtype=np.float16)
    both_nan = np.isnan(a) & np.isnan(b)
    return np.all((a.view(np.uint16) == b.view(np.uint16)) | both_nan)


def test_unpack_all_code_scale_pairs_bit_exact(smla):
    # 256 rows: row r has scale code r in every group and codes cycling through all 16
    rows = np.zeros((256, 352), dtype=np.uint8)
    codes = np.arange(512) % 16
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    rows[:, :256] = packed
    rows[:, 256:288] = np.arange(256, dtype=np.uint8)[:, None]
    rows[:, 288:] = (np.arange(256)[:, None] + np.arange(64)[None, :]) % 256
    pool = torch.from_numpy(rows).to(DEV)
    ids = np.arange(-2, 258, dtype=np.int32)          # includes invalid ids -> zero rows
    got = _np(smla.nvfp4_unpack_rows_f16(pool, torch.from_numpy(ids).to(DEV)))
    ref = oracle.nvfp4_unpack_rows_ref(rows).astype(np.float16)
    assert _same_f16(got[2:258], ref)
    assert np.all(got[:2].view(np.uint16) == 0) and np.all(got[258:].view(np.uint16) == 0)


@pytest.mark.parametrize("T,K", [(3, 100), (1, 37), (5, 1021)])
def test_stage_fp8_bit_exact(smla, T, K):
    rng = np.random.default_rng(5 + T)
    src = _edge_rows(rng, 300)
    src[3:5] = rng.standard_normal((2, 576)).astype(np.float16)   # keep staged values < 448
    # group scales around the E4M3 subnormal range: staged values land on the subnormal grid
    src[6:60] = (rng.standard_normal((54, 576)) * rng.choice([0.004, 0.01, 0.02, 0.05], size=(54, 1))
                 ).astype(np.float16)
    rows = oracle.nvfp4_pack_rows_ref(src)
    idx = rng.integers(-1, 310, size=(T, K)).astype(np.int32)      # ids >= 300 lie outside the pool
    _say("stage: T", T, "K", K)
    staged = _np(smla.nvfp4_stage_fp8(torch.from_numpy(rows).to(DEV), torch.from_numpy(idx).to(DEV)))
    ref = oracle.fp8_stage_rows_ref(rows)
    valid = (idx >= 0) & (idx < 300)
    exp = np.where(valid[..., None], ref[np.where(valid, idx, 0)], np.uint8(0))
    bad = np.argwhere(np.any(staged != exp, axis=2))
    assert bad.size == 0, f"{len(bad)} entries differ, first (t, j) = {tuple(bad[0])}, row {idx[tuple(bad[0])]}"
    mag = ref[6:60] & 0x7F
    assert ((mag > 0) & (mag < 8)).any()   # subnormal E4M3 codes occur


# ----------------------------------------------------------------------------- decode

def _setup(T, H, N, K, empty_frac, seed):
    wl = W.custom(T=T, H=H, pool_rows=N, topk=K, empty_frac=empty_frac, seed=seed)
    src = W.pool_source(wl)
    q = W.queries(wl)
    idx = W.index_lists(wl)
    return wl, src, q, idx


def _run_decode(smla, q, pool, idx, scale, num_splits=0):
    out, lse = smla.sparse_mla_decode(torch.from_numpy(q).to(DEV), pool, torch.from_numpy(idx).to(DEV),
                                      scale, num_splits=num_splits)
    return _np(out), _np(lse)


SMALL = [  # T, H, N, K, empty_frac, seed
    (1, 16, 300, 2048, 0.1, 1),     # K > N: repeated... no, distinct up to N then empties
    (3, 16, 5000, 2048, 0.15, 2),
    (5, 16, 4000, 700, 0.0, 3),     # ragged last chunk
    (2, 32, 3000, 130, 0.3, 4),     # two head groups, 3 chunks
    (4, 64, 2000, 64, 0.0, 5),      # exactly one chunk
    (3, 16, 900, 65, 0.5, 6),       # one full chunk plus one entry
    (2, 16, 100, 1, 0.0, 7),        # a single entry
    (6, 128, 3000, 256, 0.2, 8),
    (5, 64, 4000, 700, 0.1, 9),     # 64-head blocks, ragged last chunk
    (3, 192, 3000, 1000, 0.3, 10),  # three 64-head blocks
]


@pytest.mark.parametrize("T,H,N,K,ef,seed", SMALL)
def test_decode_matches_oracle(smla, T, H, N, K, ef, seed):
    _say("decode case", T, H, N, K, ef, seed)
    wl, src, q, idx = _setup(T, H, N, K, ef, seed)
    pool = build_device_pool(src, DEV)
    out, lse = _run_decode(smla, q, pool, idx, wl.softmax_scale)
    ref_out, ref_lse = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, wl.softmax_scale)
    assert_parity(out, lse, ref_out, ref_lse, f"T{T} H{H} K{K}")


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 8, 17, 40, 56, 1000])
def test_decode_every_split_count(smla, splits):
    _say("splits", splits)
    wl, src, q, idx = _setup(7, 16, 6000, 1000, 0.1, 11)
    pool = build_device_pool(src, DEV)
    out, lse = _run_decode(smla, q, pool, idx, wl.softmax_scale, num_splits=splits)
    ref_out, ref_lse = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, wl.softmax_scale)
    assert_parity(out, lse, ref_out, ref_lse, f"splits {splits}")


@pytest.mark.parametrize("splits", [6, 10, 12, 24])
def test_decode_every_split_count_32_heads(smla, splits):
    # 32 tiles per token, so these give merges of 2 .. 9 splits
    _say("splits 32 heads", splits)
    wl, src, q, idx = _setup(3, 32, 5000, 2048, 0.05, 19)
    pool = build_device_pool(src, DEV)
    out, lse = _run_decode(smla, q, pool, idx, wl.softmax_scale, num_splits=splits)
    ref_out, ref_lse = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, wl.softmax_scale)
    assert_parity(out, lse, ref_out, ref_lse, f"32 heads splits {splits}")


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 20, 30, 1000])
def test_decode_every_split_count_64_heads(smla, splits):
    _say("splits 64 heads", splits)
    wl, src, q, idx = _setup(5, 64, 6000, 900, 0.1, 18)
    pool = build_device_pool(src, DEV)
    out, lse = _run_decode(smla, q, pool, idx, wl.softmax_scale, num_splits=splits)
    ref_out, ref_lse = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, wl.softmax_scale)
    assert_parity(out, lse, ref_out, ref_lse, f"64 heads splits {splits}")


@pytest.mark.parametrize("H", [16, 64])
def test_all_empty_tokens_and_split_segments(smla, H):
    _say("empties", H)
    wl, src, q, idx = _setup(6, H, 3000, 512, 0.0, 12)
    idx[1, :] = -1                       # whole list empty
    idx[3, 100:] = -1                    # later chunks of a list empty
    idx[4, :300] = -1                    # early chunks empty
    idx[5, ::2] = 3000 + 7               # out-of-range entries count as empty
    pool = build_device_pool(src, DEV)
    for splits in (1, 4, 9, 0):
        out, lse = _run_decode(smla, q, pool, idx, wl.softmax_scale, num_splits=splits)
        ref_idx = idx.copy()
        ref_idx[ref_idx >= 3000] = -1
        ref_out, ref_lse = oracle.sparse_mla_decode_ref(q, OracleRows(src), ref_idx, wl.softmax_scale)
        assert_parity(out, lse, ref_out, ref_lse, f"empties splits {splits}")
        assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("H", [16, 64])
def test_identical_rows_give_the_latent_bit_exact(smla, H):
    _say("identical rows", H)
    wl, src, q, _ = _setup(2, H, 64, 64, 0.0, 13)
    pool = build_device_pool(src, DEV)
    idx = np.full((2, 2048), -1, dtype=np.int32)
    idx[0, :1500] = 17
    idx[1, 5::3] = 42
    out, lse = _run_decode(smla, q, pool, idx, wl.softmax_scale, num_splits=1)
    rows = oracle.nvfp4_pack_rows_ref(src[[17, 42]])
    V = oracle.nvfp4_unpack_rows_ref(rows)[:, :512].astype(np.float16)
    assert np.array_equal(out[0], np.broadcast_to(V[0], out[0].shape))
    assert np.array_equal(out[1], np.broadcast_to(V[1], out[1].shape))
    K = oracle.nvfp4_unpack_rows_ref(rows)
    s0 = wl.softmax_scale * (q[0].astype(np.float64) @ K[0])
    assert np.max(np.abs(lse[0] - (s0 + np.log(1500)))) < 1e-3


def test_permutation_and_padding_invariance(smla):
    wl, src, q, idx = _setup(4, 16, 8000, 1024, 0.0, 14)
    pool = build_device_pool(src, DEV)
    out1, lse1 = _run_decode(smla, q, pool, idx, wl.softmax_scale)
    rng = np.random.default_rng(0)
    perm = np.stack([rng.permutation(1024) for _ in range(4)])
    out2, lse2 = _run_decode(smla, q, pool, np.take_along_axis(idx, perm, 1), wl.softmax_scale)
    pad = np.full((4, 2048), -1, dtype=np.int32)
    for t in range(4):
        pad[t, np.sort(rng.choice(2048, 1024, replace=False))] = idx[t]
    out3, lse3 = _run_decode(smla, q, pool, pad, wl.softmax_scale)
    scale = np.max(np.abs(out1.astype(np.float64)))
    for o, l in ((out2, lse2), (out3, lse3)):
        assert np.max(np.abs(o.astype(np.float64) - out1)) <= 2e-3 * scale
        assert np.max(np.abs(l - lse1)) <= 1e-4


def test_deterministic(smla):
    wl, src, q, idx = _setup(9, 32, 5000, 2048, 0.05, 15)
    pool = build_device_pool(src, DEV)
    a = _run_decode(smla, q, pool, idx, wl.softmax_scale)
    b = _run_decode(smla, q, pool, idx, wl.softmax_scale)
    assert np.array_equal(a[0].view(np.uint16), b[0].view(np.uint16)) and np.array_equal(a[1], b[1])


def test_poisoned_memory_is_never_read(smla):
    # every pool row not in any list, and a guard block of rows, hold NaN scales / rope;
    # results must match a clean pool bit for bit
    wl, src, q, idx = _setup(5, 16, 4000, 1500, 0.2, 16)
    pool = build_device_pool(src, DEV)
    clean = _run_decode(smla, q, pool, idx, wl.softmax_scale)
    used = np.unique(idx[idx >= 0])
    poison = np.setdiff1d(np.arange(4000), used)
    big = torch.full((4100, 352), 0x7F, dtype=torch.uint8, device=DEV)   # guard rows 0..99
    big[100:] = pool
    big[100 + torch.from_numpy(poison).to(DEV)] = 0x7F
    view = big[100:]
    dirty = _run_decode(smla, q, view, idx, wl.softmax_scale)
    assert np.array_equal(clean[0].view(np.uint16), dirty[0].view(np.uint16))
    assert np.array_equal(clean[1], dirty[1])


def test_workspace_is_left_clean_for_reuse(smla):
    wl, src, q, idx = _setup(11, 16, 6000, 2048, 0.1, 17)
    pool = build_device_pool(src, DEV)
    ws = smla.make_workspace(11, 16, 2048, 40, DEV)
    qd, idd = torch.from_numpy(q).to(DEV), torch.from_numpy(idx).to(DEV)
    r1 = smla.sparse_mla_decode(qd, pool, idd, wl.softmax_scale, num_splits=40, workspace=ws)
    r1 = (_np(r1[0]), _np(r1[1]))
    for _ in range(3):
        r2 = smla.sparse_mla_decode(qd, pool, idd, wl.softmax_scale, num_splits=40, workspace=ws)
    assert np.array_equal(r1[0].view(np.uint16), _np(r2[0]).view(np.uint16))
    from sparse_mla_decode_04_amd.binding import decode_workspace_bytes
    nb = decode_workspace_bytes(11, 16, 2048, 40)
    cnt_off = nb - 256                      # the [HG][T] counters fill the last 256-byte block
    cnt = _np(ws[cnt_off:cnt_off + 4 * 11]).view(np.int32)
    assert np.all(cnt == 0)


def _early_count_ranges(T, K, G):
    """Ranges that start inside a token of four or more tiles and finish their part of it three
    or more tiles before their own end: (range, tiles, tiles to the part's end) for each.
    Range w covers tiles [w*C // G, (w+1)*C // G) of the T*cpt tiles."""
    cpt = -(-K // 64)
    C = T * cpt
    out = []
    for w in range(G):
        lo, hi = w * C // G, (w + 1) * C // G
        t = lo // cpt
        first_end = min(hi - lo, (t + 1) * cpt - lo)
        starts_inside = lo > t * cpt or hi < (t + 1) * cpt
        if cpt >= 4 and starts_inside and first_end <= hi - lo - 3:
            out.append((w, hi - lo, first_end))
    return out


@pytest.mark.parametrize("T,H,K,splits", [(9, 16, 250, 7), (9, 16, 250, 8), (9, 48, 250, 10),
                                          (11, 16, 200, 12), (7, 16, 1000, 25)])
def test_decode_ranges_that_count_their_first_token_early(smla, T, H, K, splits):
    # Stream-K split counts (not a multiple of T) under which a range that starts inside a token
    # counts itself for that token while it still has tiles of the next: four tiles per token
    # with a ragged last tile, and a range whose first part ends exactly three tiles before its
    # last.  Repeated launches on one workspace also check that the counters return to zero.
    early = _early_count_ranges(T, K, splits)
    assert splits % T != 0 and any(n - e == 3 for _, n, e in early), early
    _say("early count", T, H, K, splits, early)
    wl, src, q, idx = _setup(T, H, 7000, K, 0.1, 31 + splits)
    pool = build_device_pool(src, DEV)
    ref_out, ref_lse = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, wl.softmax_scale)
    ws = smla.make_workspace(T, H, K, splits, DEV)
    qd, idd = torch.from_numpy(q).to(DEV), torch.from_numpy(idx).to(DEV)
    for rep in range(3):
        out, lse = smla.sparse_mla_decode(qd, pool, idd, wl.softmax_scale, num_splits=splits, workspace=ws)
        assert_parity(_np(out), _np(lse), ref_out, ref_lse, f"early count splits {splits} rep {rep}")
    from sparse_mla_decode_04_amd.binding import decode_workspace_bytes
    nb = decode_workspace_bytes(T, H, K, splits)
    cnt = _np(ws[nb - 256:nb - 256 + 4 * T * (H // 16)]).view(np.int32)
    assert np.all(cnt == 0)


# ----------------------------------------------------------------------------- combine

def test_combine_matches_oracle(smla):
    rng = np.random.default_rng(21)
    T, S, H = 5, 7, 32
    po = rng.standard_normal((T, S, H, 512)).astype(np.float32)
    pl = (rng.standard_normal((T, S, H)) * 3).astype(np.float32)
    pl[0, 2:, :] = -np.inf
    pl[1, :, :5] = -np.inf           # all splits empty for some heads
    out, lse = smla.sparse_mla_combine(torch.from_numpy(po).to(DEV), torch.from_numpy(pl).to(DEV))
    ref_o, ref_l = oracle.lse_combine_ref(np.moveaxis(po, 1, 0), np.moveaxis(pl, 1, 0))
    assert_parity(_np(out), _np(lse), ref_o.astype(np.float16), ref_l, "combine")
    assert np.all(_np(out)[1, :5] == 0)


# ----------------------------------------------------------------------------- staged variant

@pytest.mark.parametrize("T,H,K,ef,splits", [
    (4, 16, 1000, 0.1, 0),
    (4, 64, 1000, 0.1, 0),     # 64-head blocks: the role-specialised kernel
    (5, 64, 700, 0.2, 3),      # ragged last tile, ranges across tokens
    (3, 128, 2048, 0.05, 0),
    (2, 192, 300, 0.3, 1000),  # three head blocks, one tile per workgroup
])
def test_staged_variant_matches_staged_oracle(smla, T, H, K, ef, splits):
    _say("staged", T, H, K, ef, splits)
    wl, src, q, idx = _setup(T, H, 3000, K, ef, 22 + H + splits)
    pool = build_device_pool(src, DEV)
    idd = torch.from_numpy(idx).to(DEV)
    staged = smla.nvfp4_stage_fp8(pool, idd)
    out, lse = smla.sparse_mla_decode_fp8rows(torch.from_numpy(q).to(DEV), staged, idd, 3000, wl.softmax_scale,
                                              num_splits=splits)
    ref_o, ref_l = oracle.sparse_mla_decode_fp8rows_ref(q, OracleRows(src), idx, wl.softmax_scale)
    assert_parity(_np(out), _np(lse), ref_o, ref_l, f"staged T{T} H{H} K{K} splits {splits}")

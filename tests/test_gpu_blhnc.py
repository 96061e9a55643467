"""GPU parity of the block-major multi-layer cache ([block][layer][row in block][352 bytes];
the BLHNC layout of "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily"),
called through the C ABI, against the CPU oracle:
  * nvfp4_pack_rows_blhnc bit-exact against the oracle's row writer placed by the oracle's
    block-major layout (untouched rows keep their bytes);
  * blhnc_copy_blocks bit-exact against the oracle's segment copy (gather into a send
    buffer, scatter into free blocks, skipped pairs, layer-major segments);
  * sparse_mla_decode_blhnc within the decode tolerance (max |out - ref| <= 2e-3 max |ref|,
    |lse - ref| <= 1e-3, -inf exactly where the oracle has it) against the oracle's decode of
    the same layer, for block sizes 1 to 64, head blocks of 16, 32 and 64, ragged tails,
    empty and out-of-range entries and every kind of split; and bit-identical to
    sparse_mla_decode over the same layer kept layer-major; at the full size of the
    264-token workload on sampled tokens."""

import sys

import numpy as np
import pytest

import oracle
from sparse_mla_decode_04_amd import workloads as W
from helpers import OracleRows, assert_parity, pool_source_all

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


def _layer_sources(wl, L):
    """fp16 [L, N, 576]: layer 0 is the workload's pool source, layer l > 0 the same rows
    rotated by 97 * l rows and negated on odd layers (different content per layer)."""
    src = W.pool_source(wl)
    out = [src]
    for l in range(1, L):
        s = np.roll(src, 97 * l, axis=0)
        out.append(-s if l % 2 else s)
    return np.stack(out)


def _device_blocked(smla, srcs, B, chunk=65536):
    """Pack every layer's source rows into a device block-major pool."""
    L, N, _ = srcs.shape
    pool = torch.zeros((N // B, L, B, 352), dtype=torch.uint8, device=DEV)
    for l in range(L):
        for a in range(0, N, chunk):
            b = min(N, a + chunk)
            s = torch.from_numpy(np.ascontiguousarray(srcs[l, a:b])).to(DEV)
            smla.nvfp4_pack_rows_blhnc(s, torch.arange(a, b, dtype=torch.int32, device=DEV), pool, l)
    return pool


def test_blhnc_pack_bit_exact(smla):
    _say("blhnc pack")
    rng = np.random.default_rng(21)
    L, N, B, n = 3, 256, 16, 200
    src = (rng.standard_normal((L, n, 576)) * np.exp(rng.uniform(-8, 6, (L, n, 576)))).astype(np.float16)
    pool = torch.full((N // B, L, B, 352), 0x5A, dtype=torch.uint8, device=DEV)
    expect_layers = np.full((L, N, 352), 0x5A, dtype=np.uint8)
    for l in range(L):
        slots = rng.permutation(N)[:n].astype(np.int32)
        slots[3], slots[4] = -1, N + 5              # skipped
        smla.nvfp4_pack_rows_blhnc(torch.from_numpy(src[l]).to(DEV), torch.from_numpy(slots).to(DEV), pool, l)
        ok = (slots >= 0) & (slots < N)
        expect_layers[l, slots[ok]] = oracle.nvfp4_pack_rows_ref(src[l][ok])
    assert np.array_equal(_np(pool), oracle.blocked_pool_ref(expect_layers, B))


def test_blhnc_copy_blocks_bit_exact(smla):
    _say("blhnc copy")
    rng = np.random.default_rng(22)
    nb, L, B = 40, 5, 8
    host = rng.integers(0, 256, size=(nb, L, B, 352), dtype=np.uint8)
    pool = torch.from_numpy(host).to(DEV)
    # gather a request's blocks (some ids out of range) into a contiguous send buffer
    ids = rng.permutation(nb)[:17].astype(np.int32)
    ids[2], ids[9] = -3, nb
    send = torch.full((17, L, B, 352), 0xEE, dtype=torch.uint8, device=DEV)
    smla.blhnc_copy_blocks(pool, send, src_ids=torch.from_numpy(ids).to(DEV))
    exp = oracle.copy_blocks_ref(host, np.full((17, L, B, 352), 0xEE, dtype=np.uint8), src_ids=ids)
    assert np.array_equal(_np(send), exp)
    # scatter the send buffer into free blocks of another pool
    dst_ids = rng.permutation(nb)[:17].astype(np.int32)
    dst_ids[5] = -1
    recv = torch.zeros((nb, L, B, 352), dtype=torch.uint8, device=DEV)
    smla.blhnc_copy_blocks(send, recv, dst_ids=torch.from_numpy(dst_ids).to(DEV))
    exp2 = oracle.copy_blocks_ref(exp, np.zeros((nb, L, B, 352), dtype=np.uint8), dst_ids=dst_ids)
    assert np.array_equal(_np(recv), exp2)
    # a layer-major cache moves the same rows as one segment per (block, layer)
    lm = torch.from_numpy(np.ascontiguousarray(host.transpose(1, 0, 2, 3))).to(DEV)   # [L, nb, B, 352]
    segs = lm.view(L * nb, B, 352)
    want = [3, 11, 0]
    seg_ids = np.array([l * nb + b for b in want for l in range(L)], dtype=np.int32)
    out = torch.zeros((len(seg_ids), B, 352), dtype=torch.uint8, device=DEV)
    smla.blhnc_copy_blocks(segs, out, src_ids=torch.from_numpy(seg_ids).to(DEV))
    assert np.array_equal(_np(out).reshape(len(want), L, B, 352), host[want])
    # pieces past one workgroup's chunk: segments of 40 KiB
    big = rng.integers(0, 256, size=(6, 40960), dtype=np.uint8)
    dbig = torch.zeros((6, 40960), dtype=torch.uint8, device=DEV)
    smla.blhnc_copy_blocks(torch.from_numpy(big).to(DEV), dbig, src_ids=torch.tensor([5, 4, 3, 2, 1, 0],
                                                                                      dtype=torch.int32,
                                                                                      device=DEV))
    assert np.array_equal(_np(dbig), big[::-1])


@pytest.mark.parametrize("T,H,N,K,B,layer,splits", [
    (5, 16, 4096, 1000, 16, 1, 0),
    (5, 16, 4096, 1000, 1, 2, 7),
    (5, 16, 4096, 1000, 64, 0, 1),
    (4, 32, 3072, 777, 4, 2, 0),
    (3, 64, 2048, 2048, 32, 1, 0),
    (2, 128, 2048, 300, 8, 2, 5),
    (6, 16, 1024, 64, 2, 1, 1000),     # one tile per workgroup
])
def test_blhnc_decode_matches_oracle(smla, T, H, N, K, B, layer, splits):
    _say("blhnc decode", T, H, N, K, B, layer, splits)
    L = 3
    wl = W.custom(T=T, H=H, pool_rows=N, topk=K, empty_frac=0.1, seed=300 + K + B)
    srcs = _layer_sources(wl, L)
    q, idx = W.queries(wl), W.index_lists(wl)
    rng = np.random.default_rng(K + B)
    idx[rng.random(idx.shape) < 0.02] = N + 3       # out of range: empty
    ref_idx = idx.copy()
    ref_idx[ref_idx >= N] = -1
    pool = _device_blocked(smla, srcs, B)
    dq, didx = torch.from_numpy(q).to(DEV), torch.from_numpy(idx).to(DEV)
    out, lse = smla.sparse_mla_decode_blhnc(dq, pool, layer, didx, wl.softmax_scale, num_splits=splits)
    blocked_ref = oracle.blocked_pool_ref(np.stack([oracle.nvfp4_pack_rows_ref(s) for s in srcs]), B)
    ref_o, ref_l = oracle.sparse_mla_decode_blhnc_ref(q, blocked_ref, layer, ref_idx, wl.softmax_scale)
    assert_parity(_np(out), _np(lse), ref_o, ref_l, f"blhnc T{T} H{H} K{K} B{B} layer{layer}")
    # the same kernel over the layer kept layer-major gives the same bits
    flat = torch.zeros((N, 352), dtype=torch.uint8, device=DEV)
    smla.nvfp4_pack_rows(torch.from_numpy(srcs[layer]).to(DEV), torch.arange(N, dtype=torch.int32, device=DEV),
                         flat)
    o2, l2 = smla.sparse_mla_decode(dq, flat, didx, wl.softmax_scale, num_splits=splits)
    assert np.array_equal(_np(out).view(np.uint16), _np(o2).view(np.uint16))
    assert np.array_equal(_np(lse), _np(l2))


def test_blhnc_decode_full_size(smla):
    wl = W.WORKLOADS[4]
    L, B = 2, 16
    _say(f"blhnc config 4 {wl.name}: T={wl.T} H={wl.H} pool={wl.pool_rows} layers={L} B={B}")
    src = pool_source_all(wl)
    pool = torch.zeros((wl.pool_rows // B, L, B, 352), dtype=torch.uint8, device=DEV)
    other = np.roll(src, 1, axis=0)                  # layer 0 holds different rows
    for l, s_all in ((0, other), (1, src)):
        for a in range(0, wl.pool_rows, 262144):
            b = min(wl.pool_rows, a + 262144)
            smla.nvfp4_pack_rows_blhnc(torch.from_numpy(np.ascontiguousarray(s_all[a:b])).to(DEV),
                                       torch.arange(a, b, dtype=torch.int32, device=DEV), pool, l)
    q, idx = W.queries(wl), W.index_lists(wl)
    out, lse = smla.sparse_mla_decode_blhnc(torch.from_numpy(q).to(DEV), pool, 1, torch.from_numpy(idx).to(DEV),
                                            wl.softmax_scale)
    out, lse = _np(out), _np(lse)
    rng = np.random.default_rng(104)
    toks = sorted({0, wl.T - 1} | set(rng.choice(wl.T, size=4, replace=False).tolist()))
    ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, wl.softmax_scale, tokens=toks)
    oe, le = assert_parity(out[toks], lse[toks], ref_o, ref_l, "blhnc config 4")
    assert np.all(np.isfinite(out))
    _say(f"blhnc config 4: tokens {toks} out_err {oe:.2e} lse_err {le:.2e}")

"""The decode and the cache write captured in a HIP graph (how a serving loop launches
them): every replay, with eager work and synchronizations between replays, must equal
the eager launch bit for bit, and the eager launch is checked against the oracle within
the decode tolerance.  Covers a split (in-launch merge, counters the launch leaves at
zero) and an unsplit shape, 16 and 64 heads."""

import sys

import numpy as np
import pytest

import oracle
from sparse_mla_decode_04_amd import workloads as W
from helpers import OracleRows, assert_parity, build_device_pool

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def smla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_decode_04_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("T,H,N,K,splits", [(9, 16, 6000, 1500, 0), (9, 16, 6000, 1500, 1), (3, 64, 3000, 700, 0)])
def test_graph_replays_equal_eager(smla, T, H, N, K, splits):
    print("graph", T, H, N, K, splits, file=sys.stderr, flush=True)
    wl = W.custom(T=T, H=H, pool_rows=N, topk=K, empty_frac=0.1, seed=500 + K + splits)
    src, q, idx = W.pool_source(wl), W.queries(wl), W.index_lists(wl)
    pool = build_device_pool(src, DEV)
    new = np.random.default_rng(7).standard_normal((32, 576)).astype(np.float16)
    slots = np.random.default_rng(8).permutation(N)[:32].astype(np.int32)
    src2 = src.copy()
    src2[slots] = new
    q_d, idx_d = torch.from_numpy(q).to(DEV), torch.from_numpy(idx).to(DEV)
    new_d, slots_d = torch.from_numpy(new).to(DEV), torch.from_numpy(slots).to(DEV)
    out = torch.empty((T, H, 512), dtype=torch.float16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = smla.make_workspace(T, H, K, splits)

    def step():
        smla.nvfp4_pack_rows(new_d, slots_d, pool)
        smla.sparse_mla_decode(q_d, pool, idx_d, wl.softmax_scale, out, lse, splits, ws)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src2), idx, wl.softmax_scale)
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "eager")
    e_out, e_lse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
        step()
    for r in range(4):
        out.fill_(float("nan"))
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, e_out) and torch.equal(lse, e_lse), f"replay {r}"
        step()                                   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, e_out)

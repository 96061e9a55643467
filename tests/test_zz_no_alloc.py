"""GPU check of sparse_mla_decode_noalloc (the decode entry point that allocates nothing
and keeps its split partials in the library's own scratch), called through the C ABI:
its output equals sparse_mla_decode's bit for bit on the same inputs and split count,
and is within tolerance of the oracle, on two calls in a row, the second with a smaller
input (the scratch keeps the first call's contents); a shape needing more scratch than
the library holds returns SMLA_ERR_WORKSPACE."""

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


CASES = [  # T, H, N, K, empty_frac, seed, splits: the second case of each pair is smaller
    ((6, 64, 5000, 2048, 0.1, 91, 12), (3, 16, 3000, 700, 0.2, 92, 5)),
    ((9, 16, 6000, 2048, 0.05, 93, 0), (2, 128, 2000, 300, 0.0, 94, 3)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_decode_twice(smla, first, second):
    for T, H, N, K, ef, seed, splits in (first, second):
        _say("noalloc case", T, H, N, K, ef, seed, splits)
        wl = W.custom(T=T, H=H, pool_rows=N, topk=K, empty_frac=ef, seed=seed)
        src, q, idx = W.pool_source(wl), W.queries(wl), W.index_lists(wl)
        pool = build_device_pool(src, DEV)
        q_d, idx_d = torch.from_numpy(q).to(DEV), torch.from_numpy(idx).to(DEV)
        ref = smla.sparse_mla_decode(q_d, pool, idx_d, wl.softmax_scale, num_splits=splits)
        got = smla.sparse_mla_decode_noalloc(q_d, pool, idx_d, wl.softmax_scale, num_splits=splits)
        torch.cuda.synchronize()
        assert np.array_equal(_np(got[0]).view(np.uint16), _np(ref[0]).view(np.uint16)), "out differs"
        assert np.array_equal(_np(got[1]), _np(ref[1])), "lse differs"
        ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, wl.softmax_scale)
        assert_parity(_np(got[0]), _np(got[1]), ref_o, ref_l, f"noalloc T{T} H{H} K{K}")


def test_noalloc_rejects_shapes_beyond_its_scratch(smla):
    from sparse_mla_decode_04_amd.binding import SmlaError, decode_workspace_bytes
    T, H, K = 64, 128, 2048
    splits = 4096        # 2 head blocks x 4096 ranges x 2 slots x 64 heads x 2 KiB > 80 MiB
    assert decode_workspace_bytes(T, H, K, splits) > 80 << 20
    q = torch.zeros((T, H, 576), dtype=torch.float16, device=DEV)
    pool = torch.zeros((16, 352), dtype=torch.uint8, device=DEV)
    idx = torch.full((T, K), -1, dtype=torch.int32, device=DEV)
    with pytest.raises(SmlaError, match="WORKSPACE"):
        smla.sparse_mla_decode_noalloc(q, pool, idx, 0.1, num_splits=splits)

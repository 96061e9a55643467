"""Parity at the five workloads' full sizes, in the launch configuration the
benchmark times (automatic split count): the whole pool is written by
nvfp4_pack_rows and a seeded sample of its rows is checked byte for byte against
the oracle's row writer; every token's decode runs on the GPU and a seeded sample
of tokens (plus the first and the last) is checked against the oracle."""

import sys
import time

import numpy as np
import pytest

import oracle
from sparse_mla_decode_04_amd import workloads as W
from helpers import OracleRows, assert_parity, build_device_pool, pool_source_all

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda"
N_TOKENS_CHECKED = 6


@pytest.fixture(scope="module")
def smla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_decode_04_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_parity(smla, cfg):
    wl = W.WORKLOADS[cfg]
    t0 = time.time()
    print(f"config {cfg} {wl.name}: T={wl.T} H={wl.H} pool={wl.pool_rows}", file=sys.stderr, flush=True)
    src = pool_source_all(wl)
    pool = build_device_pool(src, DEV)
    new, slots = W.new_rows(wl)
    if len(slots):   # the cache write of this workload, through the library's row writer
        smla.nvfp4_pack_rows(torch.from_numpy(new).to(DEV), torch.from_numpy(slots).to(DEV), pool)
    q = W.queries(wl)
    idx = W.index_lists(wl)
    out, lse = smla.sparse_mla_decode(torch.from_numpy(q).to(DEV), pool, torch.from_numpy(idx).to(DEV),
                                      wl.softmax_scale)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    rng = np.random.default_rng(cfg)
    # pack: sampled rows (and every new row) byte-exact
    sample = rng.choice(wl.pool_rows, size=min(wl.pool_rows, 4096), replace=False)
    sample = np.union1d(sample, slots)
    got = pool[torch.from_numpy(sample).to(DEV)].cpu().numpy()
    ref = oracle.nvfp4_pack_rows_ref(src[sample])
    assert np.array_equal(got, ref), f"pack differs on {int(np.sum(np.any(got != ref, axis=1)))} rows"
    # decode: sampled tokens
    toks = sorted(set([0, wl.T - 1]) | set(rng.choice(wl.T, size=min(wl.T, N_TOKENS_CHECKED), replace=False).tolist()))
    ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, wl.softmax_scale, tokens=toks)
    oe, le = assert_parity(out[toks], lse[toks], ref_o, ref_l, f"config {cfg}")
    assert np.all(np.isfinite(out))
    print(f"config {cfg}: tokens {toks} out_err {oe:.2e} lse_err {le:.2e} ({time.time() - t0:.1f}s)",
          file=sys.stderr, flush=True)

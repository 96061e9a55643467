"""Parity at the five workloads' full sizes, in the launch configuration the
benchmark times (automatic split count).  The whole pool is written by
nvfp4_pack_rows; every row a checked token's list names, plus a seeded sample of
other rows and every newly written row, is compared byte for byte against the
oracle's row writer.  Every token's decode runs on the GPU; every token is checked
against the oracle at the 1-, 35-, 128- and 264-token workloads, and 64 seeded tokens
(plus the first and the last) at the 1,024-token one.  At the 1,024-token workload the
staged two-pass variant (FP8 rows written to HBM, then attention over them) is checked
against the staged oracle on 8 seeded tokens."""

import sys
import time

import numpy as np
import pytest

import oracle
from sparse_mla_decode_04_amd import workloads as W
from helpers import PackedRows, assert_parity, build_device_pool, pool_source_all

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda"
ALL_TOKENS_UP_TO = 264  # workloads of at most this many tokens are checked token by token
SAMPLED_TOKENS = 64     # seeded tokens checked at the larger workload
STAGED_TOKENS = 8


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def smla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_decode_04_amd as m
    m.lib()
    return m


def _setup(smla, cfg):
    wl = W.WORKLOADS[cfg]
    src = pool_source_all(wl)
    pool = build_device_pool(src, DEV)
    new, slots = W.new_rows(wl)
    if len(slots):   # the cache write of this workload, through the library's row writer
        smla.nvfp4_pack_rows(torch.from_numpy(new).to(DEV), torch.from_numpy(slots).to(DEV), pool)
    return wl, src, pool, slots, W.queries(wl), W.index_lists(wl)


def _checked_tokens(wl, rng, n):
    if wl.T <= max(n, ALL_TOKENS_UP_TO):
        return list(range(wl.T))
    return sorted(set([0, wl.T - 1]) | set(rng.choice(wl.T, size=n, replace=False).tolist()))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_parity(smla, cfg):
    t0 = time.time()
    wl, src, pool, slots, q, idx = _setup(smla, cfg)
    _say(f"config {cfg} {wl.name}: T={wl.T} H={wl.H} pool={wl.pool_rows} ({time.time() - t0:.1f}s)")
    out, lse = smla.sparse_mla_decode(torch.from_numpy(q).to(DEV), pool, torch.from_numpy(idx).to(DEV),
                                      wl.softmax_scale)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(out))
    rng = np.random.default_rng(cfg)
    toks = _checked_tokens(wl, rng, SAMPLED_TOKENS)
    sample = rng.choice(wl.pool_rows, size=min(wl.pool_rows, 4096), replace=False)
    rows = PackedRows(src, np.concatenate([idx[toks].ravel(), sample, slots]))
    _say(f"config {cfg}: oracle rows {len(rows.ids)} ({time.time() - t0:.1f}s)")
    # pack: every prepared row byte-exact
    got = pool[torch.from_numpy(rows.ids).to(DEV)].cpu().numpy()
    bad = np.any(got != rows.rows, axis=1)
    assert not np.any(bad), f"pack differs on {int(bad.sum())} rows, e.g. {rows.ids[bad][:5]}"
    ref_o, ref_l = oracle.sparse_mla_decode_ref(q, rows, idx, wl.softmax_scale, tokens=toks)
    oe, le = assert_parity(out[toks], lse[toks], ref_o, ref_l, f"config {cfg}")
    _say(f"config {cfg}: {len(toks)} tokens out_err {oe:.2e} lse_err {le:.2e} ({time.time() - t0:.1f}s)")


def test_staged_variant_full_size(smla):
    t0 = time.time()
    wl, src, pool, slots, q, idx = _setup(smla, 5)
    _say(f"staged, config 5: T={wl.T} H={wl.H} ({time.time() - t0:.1f}s)")
    idd = torch.from_numpy(idx).to(DEV)
    staged = smla.nvfp4_stage_fp8(pool, idd)
    out, lse = smla.sparse_mla_decode_fp8rows(torch.from_numpy(q).to(DEV), staged, idd, wl.pool_rows,
                                              wl.softmax_scale)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    del staged
    assert np.all(np.isfinite(out))
    rng = np.random.default_rng(55)
    toks = sorted(rng.choice(wl.T, size=STAGED_TOKENS, replace=False).tolist())
    rows = PackedRows(src, idx[toks].ravel())
    ref_o, ref_l = oracle.sparse_mla_decode_fp8rows_ref(q, rows, idx, wl.softmax_scale, tokens=toks)
    oe, le = assert_parity(out[toks], lse[toks], ref_o, ref_l, "staged config 5")
    _say(f"staged config 5: tokens {toks} out_err {oe:.2e} lse_err {le:.2e} ({time.time() - t0:.1f}s)")

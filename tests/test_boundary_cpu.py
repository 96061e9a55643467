"""The C-ABI library without a GPU: it loads, exports every entry point that
include/smla.h declares, and rejects bad arguments on the host (before any
launch) with the documented status codes."""

import ctypes
import os
import re

import pytest

import sparse_mla_decode_04_amd as smla
from sparse_mla_decode_04_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "smla.h")).read()
    return set(re.findall(r"SMLA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libsmla.so not built")
    return smla.lib()


def test_header_and_binding_agree():
    assert _declared() == set(binding.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings(L):
    assert L.smla_status_string(0) == b"SMLA_OK"
    assert L.smla_status_string(-3) == b"SMLA_ERR_WORKSPACE"
    assert L.smla_status_string(-99) == b"SMLA_ERR_UNKNOWN"


def test_workspace_and_split_queries(L):
    assert smla.choose_num_splits(35, 16, 2048) >= 1
    assert smla.decode_workspace_bytes(35, 16, 2048, 0) > 0
    assert smla.decode_workspace_bytes(35, 24, 2048, 0) == 0      # unsupported H
    assert smla.decode_workspace_bytes(0, 16, 2048, 0) == 0
    # one workgroup per head group owning every token: no partials needed beyond one slot
    assert smla.decode_workspace_bytes(4, 16, 2048, 1) < smla.decode_workspace_bytes(4, 16, 2048, 32)


P = ctypes.c_void_p


def _decode(L, q=16, pool=16, idx=16, T=1, H=16, topk=64, scale=0.1, out=16, lse=16, ns=0, ws=None, wsb=1 << 30):
    return L.sparse_mla_decode(P(q), P(pool), 100, P(idx), T, H, topk, scale, P(out), P(lse), ns,
                               P(ws), wsb, None)


def test_decode_argument_checks(L):
    assert _decode(L, q=None) == -1
    assert _decode(L, q=8) == -1                   # misaligned
    assert _decode(L, H=24) == -2                  # not a multiple of 16
    assert _decode(L, topk=0) == -1
    assert _decode(L, topk=70000) == -1
    assert _decode(L, ns=-1) == -1
    assert _decode(L, scale=float("nan")) == -1
    assert _decode(L, scale=float("inf")) == -1
    assert _decode(L, scale=0.0) == -1             # a zero or negative scale is rejected
    assert _decode(L, scale=-0.5) == -1
    assert _decode(L, ws=None) == -3               # workspace missing
    assert _decode(L, ws=16, wsb=10) == -3         # workspace too small
    assert _decode(L, T=0, q=None, pool=None, idx=None, out=None, lse=None) == 0   # nothing to do


def test_noalloc_decode_argument_checks(L):
    # argument errors come back before the library looks up its scratch on a device
    f = L.sparse_mla_decode_noalloc
    assert f(None, P(16), 100, P(16), 1, 16, 64, 0.1, P(16), P(16), 0, None) == -1
    assert f(P(16), P(16), 100, P(16), 1, 24, 64, 0.1, P(16), P(16), 0, None) == -2
    assert f(P(16), P(16), 100, P(16), 1, 16, 64, 0.0, P(16), P(16), 0, None) == -1
    assert f(P(16), P(16), 100, P(16), 1, 16, 0, 0.1, P(16), P(16), 0, None) == -1
    assert f(P(16), P(16), 100, P(16), 1, 16, 64, 0.1, P(16), P(16), -2, None) == -1
    assert f(None, None, 100, None, 0, 16, 64, 0.1, None, None, 0, None) == 0    # T == 0: nothing to do


def test_other_entry_points_check_arguments(L):
    assert L.nvfp4_pack_rows(None, None, 0, None, 10, None) == 0        # n == 0: no-op
    assert L.nvfp4_pack_rows(None, P(16), 3, P(16), 10, None) == -1
    assert L.nvfp4_pack_rows(P(16), P(16), -1, P(16), 10, None) == -1
    assert L.nvfp4_unpack_rows_f16(P(16), 10, None, 2, P(16), None) == -1
    assert L.sparse_mla_combine(P(16), P(16), 2, 0, 16, P(16), P(16), None) == -1
    assert L.sparse_mla_combine(P(16), P(16), 2, 2, 8, P(16), P(16), None) == -2
    assert L.nvfp4_stage_fp8(P(16), 10, P(16), 2, 0, P(16), None) == -1
    assert L.sparse_mla_decode_fp8rows(P(16), P(16), P(16), 10, 1, 16, 64, 0.1, P(16), P(16), 0,
                                       None, 0, None) == -3


def test_python_binding_rejects_host_tensors():
    import torch
    with pytest.raises((ValueError, TypeError)):
        smla.nvfp4_pack_rows(torch.zeros(2, 576, dtype=torch.float16), torch.zeros(2, dtype=torch.int32),
                             torch.zeros(4, 352, dtype=torch.uint8))


def test_grouped_entry_points_check_arguments(L):
    # union builder: tpg out of range, T not a multiple of tpg, too many entries, huge pool
    assert L.smla_group_union(P(16), 8, 64, 0, 100, 64, P(16), P(16), None) == -1
    assert L.smla_group_union(P(16), 8, 64, 5, 100, 64, P(16), P(16), None) == -1
    assert L.smla_group_union(P(16), 6, 64, 4, 100, 64, P(16), P(16), None) == -1
    assert L.smla_group_union(P(16), 8, 4096, 4, 100, 64, P(16), P(16), None) == -2
    assert L.smla_group_union(P(16), 8, 64, 4, 1 << 28, 64, P(16), P(16), None) == -2
    assert L.smla_group_union(P(16), 8, 64, 4, 100, 0, P(16), P(16), None) == -1
    assert L.smla_group_union(None, 8, 64, 4, 100, 64, P(16), P(16), None) == -1
    assert L.smla_group_union(None, 0, 64, 4, 100, 64, None, None, None) == 0      # nothing to do
    # grouped decode: tpg * H must be 64
    args = dict(q=16, pool=16, uni=16, T=8, H=16, tpg=4, U=128, out=16, lse=16)

    def dec(**kw):
        a = dict(args, **kw)
        return L.sparse_mla_decode_grouped(P(a["q"]), P(a["pool"]), 100, P(a["uni"]), a["T"], a["H"], a["tpg"],
                                           a["U"], 0.1, P(a["out"]), P(a["lse"]), 0, None, 0, None)
    assert dec(H=32) == -2
    assert dec(tpg=3, T=9) == -2
    assert dec(T=6) == -1
    assert dec(U=0) == -1
    assert dec(q=None) == -1
    assert dec() == -3                                   # workspace missing
    assert smla.grouped_workspace_bytes(264, 16, 4, 3584) > 0
    assert smla.grouped_workspace_bytes(264, 16, 3, 3584) == 0


def test_fp8pool_entry_points_check_arguments(L):
    assert L.fp8_pack_rows(None, None, 0, None, 10, None) == 0          # n == 0: no-op
    assert L.fp8_pack_rows(None, P(16), 3, P(16), 10, None) == -1
    assert L.fp8_pack_rows(P(16), P(16), 3, P(8), 10, None) == -1        # misaligned pool
    assert L.fp8_pack_rows(P(16), P(16), -1, P(16), 10, None) == -1

    def dec(pool_rows=100, H=16, q=16):
        return L.sparse_mla_decode_fp8pool(P(q), P(16), pool_rows, P(16), 2, H, 64, 0.1, P(16), P(16), 0,
                                           None, 0, None)
    assert dec(q=None) == -1
    assert dec(H=24) == -2
    assert dec() == -3                                   # workspace missing
    # 8M rows of 576 bytes exceed one buffer resource's 4 GiB range; as NVFP4 rows they fit
    assert dec(pool_rows=8_000_000) == -2
    assert L.sparse_mla_decode(P(16), P(16), 8_000_000, P(16), 2, 16, 64, 0.1, P(16), P(16), 0,
                               None, 0, None) == -3


def test_indexer_entry_point_checks_arguments(L):
    def topk(scores=16, ld=8, lengths=None, T=2, k=4, out=16, parts=0, ws=None, nb=0):
        return L.sparse_indexer_topk(P(scores), ld, P(lengths), None, T, k, P(out), parts, P(ws), nb, None)
    assert topk(scores=None, out=None, T=0) == 0           # T == 0: no-op
    assert topk(k=0) == -1                                 # k < 1
    assert topk(k=65537) == -1                             # k too large
    assert topk(ld=6) == -1                                # ld not a multiple of 4
    assert topk(scores=8) == -1                            # misaligned scores
    assert topk(scores=None) == -1
    assert topk(lengths=2) == -1                           # misaligned lengths
    assert topk(out=None) == -1                            # no output
    assert topk(parts=-1) == -1
    assert topk(parts=65) == -1                            # more workgroups per token than the split takes
    assert topk(parts=2) == -3                             # a split without a workspace
    assert topk(parts=2, ws=16, nb=16) == -3               # a workspace too small for it
    assert topk(parts=2, ws=8, nb=1 << 30) == -3           # a misaligned one


def test_indexer_workspace_query(L):
    L.smla_indexer_workspace_bytes.restype = ctypes.c_size_t
    assert L.smla_indexer_workspace_bytes(2, 8192, 4, 1) == 0          # one workgroup per token
    two = L.smla_indexer_workspace_bytes(2, 8192, 4, 2)
    assert two > 0 and two % 256 == 0
    assert L.smla_indexer_workspace_bytes(2, 8192, 4, 7) > two         # a histogram per workgroup
    assert L.smla_indexer_workspace_bytes(0, 8192, 4, 2) == 0
    assert L.smla_indexer_workspace_bytes(2, 8192, 4, 65) == 0         # invalid
    assert L.smla_indexer_workspace_bytes(2, 6, 4, 2) == 0


def test_blhnc_entry_points_check_arguments(L):
    def dec(nb=100, layers=4, layer=1, B=16, ws=None):
        return L.sparse_mla_decode_blhnc(P(16), P(16), nb, layers, layer, B, P(16), 2, 16, 64, 0.1, P(16),
                                         P(16), 0, ws, 0, None)
    assert dec(B=12) == -1                               # block size not a power of two
    assert dec(B=0) == -1
    assert dec(layer=4) == -1                            # layer past the layers
    assert dec(layer=-1) == -1
    assert dec(layers=0) == -1
    assert dec(nb=-1) == -1
    assert dec(layers=1 << 10, B=1 << 14) == -1          # stride layers * B reaches 2^24
    assert dec() == -3                                   # well formed: workspace missing
    # the whole allocation (every layer) must fit one buffer resource's byte range
    assert dec(nb=1_000_000 // 16 * 4, layers=4) == -2
    assert L.nvfp4_pack_rows_blhnc(None, None, 0, None, 10, 2, 0, 8, None) == 0          # n == 0
    assert L.nvfp4_pack_rows_blhnc(P(16), P(16), 3, P(16), 10, 2, 2, 8, None) == -1      # bad layer
    assert L.nvfp4_pack_rows_blhnc(P(16), P(16), 3, P(8), 10, 2, 0, 8, None) == -1       # misaligned pool
    assert L.nvfp4_pack_rows_blhnc(P(16), P(16), 3, P(16), 1 << 29, 2, 0, 8, None) == -2  # rows past int32
    cp = L.blhnc_copy_blocks
    assert cp(None, 0, None, None, 0, None, 0, 16, None) == 0                           # n == 0
    assert cp(P(16), 4, None, P(16), 4, None, 2, 24, None) == -1                        # not a multiple of 16
    assert cp(P(16), 4, None, P(16), 4, None, 2, 0, None) == -1
    assert cp(P(8), 4, None, P(16), 4, None, 2, 16, None) == -1                         # misaligned source
    assert cp(P(16), 4, P(2), P(16), 4, None, 2, 16, None) == -1                        # misaligned ids
    assert cp(P(16), 4, None, None, 4, None, 2, 16, None) == -1
    assert cp(P(16), 4, None, P(16), 4, None, 1 << 20, 1 << 20, None) == -2             # grid too large


def test_blhnc_decode_rejects_block_counts_that_would_wrap(L):
    # 2^60 blocks x 16 layers x 16 rows wraps 64 bits; the call must still be refused
    assert L.sparse_mla_decode_blhnc(P(16), P(16), 1 << 60, 16, 0, 16, P(16), 2, 16, 64, 0.1, P(16), P(16), 0,
                                     None, 0, None) == -2

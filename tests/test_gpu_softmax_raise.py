"""GPU parity of the FP32 online softmax when a later tile dominates ("Prime Intellect
Launches Prime Inference, Serving 600B Tokens Daily", section "Four-bit caches make room":
FP16 operands with FP32 accumulation), called through the C ABI, against the CPU oracle.

The kernels keep a per-head reference score and raise it mid-segment only when a tile
beats it by more than a slack; then they rescale the accumulator and the probabilities
already formed.  Scores a few units apart never reach that path, so these inputs make
later tiles win by a wide margin:

  * ramp: every pool row is a_r * base + noise with a_r uniform in [-8, 8], every query
    head is base + noise, so the score of row r is close to 24 * a_r for every head.
    Each list holds its rows in ascending a_r, so each tile of 64 entries beats the one
    before by about 17 log2 units.  The first three tiles of every list, and three tiles
    from entry 1,024 on, are empty: a segment (and, with two splits per token, the
    second range) starts with empty tiles and then peaks.
  * wide: N(0,1) rows and queries with softmax_scale = 1 (scores spread over about
    35 log2 units per standard deviation) in random list order.

Every decode kernel and mode is covered at several split counts: the 16-head register
kernel, the 32-head ring kernel, the 64-head role-specialised kernel (64 and 128 heads),
the 16-head ring and role-specialised variants (child processes), decode over an FP8
pool, the staged pass 2, grouped decode and decode over a block-major pool.
Tolerances: max |out - ref| <= 2e-3 max |ref|, |lse - ref| <= 1e-3."""

import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from helpers import OracleFp8Rows, OracleRows, assert_parity, build_device_fp8_pool, build_device_pool

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


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


def ramp_inputs(T, H, N, K, seed, amp=8.0, tpg=1, shared=0.0):
    """(src fp16 [N, 576], q fp16 [T, H, 576], idx int32 [T, K], scale).  Lists ascend in
    a_r; entries 0..191 and 1024..1215 are empty (when K is large enough).  With tpg > 1,
    each group of tpg tokens shares a fraction `shared` of its rows."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal(576)
    a = rng.uniform(-amp, amp, size=N)
    src = (a[:, None] * base[None, :] + 0.5 * rng.standard_normal((N, 576))).astype(np.float16)
    q = (base[None, None, :] + 0.5 * rng.standard_normal((T, H, 576))).astype(np.float16)
    nvalid = K - (192 if K > 256 else 0) - (192 if K > 1216 else 0)
    idx = np.full((T, K), -1, dtype=np.int32)
    for g in range(0, T, tpg):
        perm = rng.permutation(N)
        ns = int(shared * nvalid)
        common, pos = perm[:ns], ns
        for t in range(g, min(T, g + tpg)):
            rows = np.concatenate([common, perm[pos:pos + nvalid - ns]])
            pos += nvalid - ns
            rows = rows[np.argsort(a[rows], kind="stable")]
            slots = np.arange(K)
            if K > 256:
                slots = slots[slots >= 192]
            if K > 1216:
                slots = slots[(slots < 1024) | (slots >= 1216)]
            idx[t, slots[:nvalid]] = rows
    return src, q, idx, 1.0 / 24.0


def wide_inputs(T, H, N, K, seed):
    rng = np.random.default_rng(seed)
    src = rng.standard_normal((N, 576)).astype(np.float16)
    q = rng.standard_normal((T, H, 576)).astype(np.float16)
    idx = np.stack([rng.permutation(N)[:K] for _ in range(T)]).astype(np.int32)
    idx[rng.random(idx.shape) < 0.05] = -1
    return src, q, idx, 1.0


def _decode(smla, q, pool, idx, scale, splits):
    out, lse = smla.sparse_mla_decode(torch.from_numpy(q).to(DEV), pool, torch.from_numpy(idx).to(DEV),
                                      scale, num_splits=splits)
    return _np(out), _np(lse)


@pytest.mark.parametrize("kind", ["ramp", "wide"])
@pytest.mark.parametrize("H", [16, 32, 64, 128])
def test_decode_later_tiles_dominate(smla, kind, H):
    T, N, K = (3, 6000, 2048) if H <= 64 else (2, 6000, 2048)
    src, q, idx, scale = (ramp_inputs if kind == "ramp" else wide_inputs)(T, H, N, K, 300 + H)
    pool = build_device_pool(src, DEV)
    ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, scale)
    for splits in (1, 2, 3, 7, 0):
        _say("raise", kind, "H", H, "splits", splits)
        out, lse = _decode(smla, q, pool, idx, scale, splits)
        assert_parity(out, lse, ref_o, ref_l, f"{kind} H{H} splits {splits}")


def test_ramp_reaches_the_raise():
    # The inputs do what they are for: every list's tiles ascend by more than the kernels'
    # slack of 8 log2 units, judged from the oracle's own scores.
    src, q, idx, scale = ramp_inputs(2, 16, 6000, 2048, 316)
    from oracle.attention import dense_rows_for
    for t in range(2):
        ids = idx[t]
        tile_max = []
        for c in range(0, 2048, 64):
            v = ids[c:c + 64]
            v = v[v >= 0]
            if len(v):
                K = dense_rows_for(OracleRows(src), v)
                s = scale * (K @ q[t].astype(np.float64).T) / np.log(2.0)
                tile_max.append(s.max(axis=0))
        jumps = np.diff(np.stack(tile_max), axis=0)
        assert np.all(jumps.min(axis=1) > 8.0)


CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import numpy as np, torch
import oracle
import sparse_mla_decode_04_amd as smla
from helpers import OracleRows, assert_parity, build_device_pool
from test_gpu_softmax_raise import ramp_inputs, wide_inputs
for kind, fn in (("ramp", ramp_inputs), ("wide", wide_inputs)):
    src, q, idx, scale = fn(5, 16, 6000, 2048, 331)
    pool = build_device_pool(src, "cuda")
    ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, scale)
    for splits in (1, 2, 5, 0):
        print("variant raise", kind, "splits", splits, flush=True)
        o, l = smla.sparse_mla_decode(torch.from_numpy(q).cuda(), pool, torch.from_numpy(idx).cuda(),
                                      scale, num_splits=splits)
        assert_parity(o.cpu().numpy(), l.cpu().numpy(), ref_o, ref_l, f"{{kind}} splits {{splits}}")
print("ok", flush=True)
"""


@pytest.mark.parametrize("variant", ["ring", "ws"])
def test_variant_later_tiles_dominate(variant):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    env = dict(os.environ, SMLA_DECODE_VARIANT=variant)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=110)
    print(r.stdout[-2000:], file=sys.stderr)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.strip().endswith("ok")


@pytest.mark.parametrize("kind", ["ramp", "wide"])
@pytest.mark.parametrize("H", [16, 32, 64, 128])
def test_fp8pool_later_tiles_dominate(smla, kind, H):
    src, q, idx, scale = (ramp_inputs if kind == "ramp" else wide_inputs)(3, H, 5000, 2048, 340 + H)
    pool = build_device_fp8_pool(src, DEV)
    ref_o, ref_l = oracle.sparse_mla_decode_fp8pool_ref(q, OracleFp8Rows(src), idx, scale)
    for splits in (1, 3, 0):
        _say("fp8pool raise", kind, H, splits)
        out, lse = smla.sparse_mla_decode_fp8pool(torch.from_numpy(q).to(DEV), pool,
                                                  torch.from_numpy(idx).to(DEV), scale, num_splits=splits)
        assert_parity(_np(out), _np(lse), ref_o, ref_l, f"fp8pool {kind} H{H} splits {splits}")


@pytest.mark.parametrize("kind", ["ramp", "wide"])
@pytest.mark.parametrize("H", [16, 64])
def test_staged_later_tiles_dominate(smla, kind, H):
    src, q, idx, scale = (ramp_inputs if kind == "ramp" else wide_inputs)(3, H, 5000, 2048, 350 + H)
    pool = build_device_pool(src, DEV)
    idd = torch.from_numpy(idx).to(DEV)
    staged = smla.nvfp4_stage_fp8(pool, idd)
    ref_o, ref_l = oracle.sparse_mla_decode_fp8rows_ref(q, OracleRows(src), idx, scale)
    for splits in (1, 4, 0):
        _say("staged raise", kind, H, splits)
        out, lse = smla.sparse_mla_decode_fp8rows(torch.from_numpy(q).to(DEV), staged, idd, 5000, scale,
                                                  num_splits=splits)
        assert_parity(_np(out), _np(lse), ref_o, ref_l, f"staged {kind} H{H} splits {splits}")


@pytest.mark.parametrize("splits", [1, 3, 0])
def test_grouped_later_tiles_dominate(smla, splits):
    _say("grouped raise", splits)
    N, tpg = 12000, 4
    src, q, idx, scale = ramp_inputs(8, 16, N, 2048, 360, tpg=tpg, shared=0.75)
    pool = build_device_pool(src, DEV)
    uni, _ = smla.group_union(torch.from_numpy(idx).to(DEV), tpg, N, tpg * 2048)
    out, lse = smla.sparse_mla_decode_grouped(torch.from_numpy(q).to(DEV), pool, uni, tpg, scale,
                                              num_splits=splits)
    ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, scale)
    assert_parity(_np(out), _np(lse), ref_o, ref_l, f"grouped splits {splits}")


@pytest.mark.parametrize("H", [16, 64])
def test_blhnc_later_tiles_dominate(smla, H):
    N, L, B, layer = 6144, 3, 16, 1
    src, q, idx, scale = ramp_inputs(3, H, N, 2048, 370 + H)
    pool = torch.zeros((N // B, L, B, 352), dtype=torch.uint8, device=DEV)
    other = np.roll(src, 77, axis=0)
    for l in range(L):
        s = torch.from_numpy(np.ascontiguousarray(src if l == layer else other)).to(DEV)
        smla.nvfp4_pack_rows_blhnc(s, torch.arange(N, dtype=torch.int32, device=DEV), pool, l)
    ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, scale)
    for splits in (1, 2, 0):
        _say("blhnc raise", H, splits)
        out, lse = smla.sparse_mla_decode_blhnc(torch.from_numpy(q).to(DEV), pool, layer,
                                                torch.from_numpy(idx).to(DEV), scale, num_splits=splits)
        assert_parity(_np(out), _np(lse), ref_o, ref_l, f"blhnc H{H} splits {splits}")

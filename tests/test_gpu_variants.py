"""GPU parity of the alternative decode kernels for 16-head blocks.

The library reads SMLA_DECODE_VARIANT once per process ("ring": the LDS-ring kernel,
"ws": the role-specialised kernel; the default is the register-gather kernel), so each
variant runs in a child process that checks sparse_mla_decode against the oracle on a
small shape (several tiles, a ragged tail, empty entries) for several split counts.
"""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import numpy as np, torch
import oracle
import sparse_mla_decode_04_amd as smla
from sparse_mla_decode_04_amd import workloads as W
from helpers import OracleRows, assert_parity, build_device_pool
wl = W.custom(T=7, H=16, pool_rows=6000, topk=1000, empty_frac=0.1, seed=23)
src = W.pool_source(wl); q = W.queries(wl); idx = W.index_lists(wl)
pool = build_device_pool(src, "cuda")
ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src), idx, wl.softmax_scale)
for splits in (0, 1, 5, 40, 1000):
    print("variant case splits", splits, flush=True)
    o, l = smla.sparse_mla_decode(torch.from_numpy(q).cuda(), pool, torch.from_numpy(idx).cuda(),
                                  wl.softmax_scale, num_splits=splits)
    assert_parity(o.cpu().numpy(), l.cpu().numpy(), ref_o, ref_l, f"splits {{splits}}")
print("ok", flush=True)
"""


@pytest.mark.parametrize("variant", ["ring", "ws"])
def test_decode_variant_matches_oracle(variant):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    env = dict(os.environ, SMLA_DECODE_VARIANT=variant)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=110)
    print(r.stdout[-2000:], file=sys.stderr)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.strip().endswith("ok")

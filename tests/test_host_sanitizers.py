"""Host code of the C-ABI library under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/host_asan/driver.cpp is linked with the library's sources, host code instrumented
(device code is compiled as usual and never launched: no GPU is needed).  It sweeps every
size query over edge values of its arguments and calls every entry point with the argument
errors it must reject before any device work; a sanitizer report, a wrong status or a
crash fails the test.  This found a signed overflow in the grouped decode's head-count
check (H * tpg in 32 bits), now done in 64 bits."""

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from sparse_mla_decode_04_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "host_asan", "driver.cpp")
# sanitizers on the host side of each translation unit only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-fno-gpu-sanitize"]
FLAGS = ["-O1", "-g", "-std=c++17", f"--offload-arch={B.ARCH}", "-fno-omit-frame-pointer",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{os.path.join(ROOT, 'include')}", f"-I{B.CSRC}", *SAN]


def _asan_runtime_present():
    llvm = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(llvm):
        return False
    for v in os.listdir(llvm):
        if os.path.exists(os.path.join(llvm, v, "lib", "linux", "libclang_rt.asan-x86_64.a")):
            return True
    return False


@pytest.mark.timeout(600)
def test_host_code_under_sanitizers():
    hipcc = B._hipcc()
    if shutil.which(hipcc) is None or not _asan_runtime_present():
        pytest.skip("hipcc or the sanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as tmp:
        def cc(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            r = subprocess.run([hipcc, *FLAGS, "-c", *lang, src, "-o", obj], capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
            return obj
        srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES] + [DRIVER]
        with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            objs = list(ex.map(cc, srcs))
        exe = os.path.join(tmp, "driver")
        r = subprocess.run([hipcc, f"--offload-arch={B.ARCH}", *SAN[:4], *objs, "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
        assert "host checks passed" in r.stdout

"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every HIP source is compiled as for the product (gfx950 device code unchanged) with the
sanitizers on its host side only, linked with tests/host_sanitize_driver.cpp, and run on
the CPU: the driver calls every entry point that works on the host (validation, union and
trie building, size and plan queries, argument checks) on random and extreme inputs.  Any
memory error or undefined behaviour aborts the driver, and a failed check exits non-zero.
"""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from candidate_likelihood_scoring_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(B.HIPCC) and os.path.exists(CLANG)),
                    reason="needs hipcc and the ROCm clang")
def test_host_code_under_asan_ubsan(tmp_path):
    flags = [f for f in B.FLAGS if f not in ("-fvisibility=hidden",)]
    srcs = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        r = subprocess.run([B.HIPCC, *flags, *SAN, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv_o = str(tmp_path / "driver.o")
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c",
                        os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), "-o", drv_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = str(tmp_path / "driver")
    rocm_lib = "/opt/rocm/lib"
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", drv_o, *objs, f"-L{rocm_lib}",
                        "-lamdhip64", f"-Wl,-rpath,{rocm_lib}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               ASAN_OPTIONS="abort_on_error=0:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "all checks passed" in r.stdout
    shutil.rmtree(tmp_path, ignore_errors=True)

"""The C-ABI's host code under AddressSanitizer: test_abi.py runs in a child
process against a copy of the library whose api.cpp is built with ASan
(build_asan.py), with the matching runtime preloaded.  Every argument check,
workspace-size computation and status path that test_abi.py reaches is then
checked for out-of-bounds and use-after-free accesses on the host.  CPU only:
the calls return before any HIP call."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_asan():
    from gemm_epilogue_fusion_gemm1_amd import build_asan
    try:
        rt = build_asan.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build_asan.build_asan(verbose=False)
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", CODA_ABI_TEST_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out

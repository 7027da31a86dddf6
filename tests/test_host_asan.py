"""The C-ABI host code (validation, workspace sizing, layout arithmetic, error
strings) under AddressSanitizer: build libssa_asan.so with ASan on the host
pass only, then run tests/asan_abi_driver.py against it in a child process
with the clang ASan runtime preloaded. GPU code is not instrumented and no
kernel is launched, so no device is needed."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_abi_host_paths_under_asan():
    from block_sparse_full_amd import build
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not available")
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    lib = build.build_host_asan_library()
    env = dict(os.environ)
    # ASan must come first among preloaded libraries; keep whatever is there after it
    env["LD_PRELOAD"] = ":".join(x for x in (rt, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=66"
    env["HIP_VISIBLE_DEVICES"] = ""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "asan_abi_driver.py"), lib],
                       capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "host paths driven: 32" in r.stdout, out[-2000:]

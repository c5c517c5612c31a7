"""The host code of libpa (argument validation, split planning, prefix
detection, table checks) under AddressSanitizer and
UndefinedBehaviorSanitizer: a g++ build of pa_host.cpp and pa_api.cpp with
the launches replaced by stand-ins (build_host_sanitized), loaded in a child
process with the ASan runtime preloaded, runs the C-ABI tests and the
prefix-detection tests.  Any sanitizer report fails the child."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_and_host_planners_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from paged_kv_decode_02_amd import build

    lib = build.build_host_sanitized(str(tmp_path / "libpa_host_asan.so"))
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not asan or not os.path.exists(asan):
        pytest.skip("libasan not found")
    env = dict(os.environ, PA_LIB=lib, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", PYTHONPATH=ROOT)
    # the child loads the sanitized library, not the in-tree one
    probe = ("import ctypes; from paged_kv_decode_02_amd import pa; assert pa.LIB_PATH == %r; pa.load(); "
             "ctypes.CDLL(None).__asan_init; print('sanitized library loaded')" % lib)
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, cwd=str(tmp_path),
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_prefix_groups.py")],
                       env=env, capture_output=True, text=True, cwd=str(tmp_path), timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out

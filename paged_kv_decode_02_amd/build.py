"""Build libpa.so in-tree with hipcc for gfx950.

    python -m paged_kv_decode_02_amd.build

Every call compiles from source (no staleness check).  The library is placed
next to this file, where the Python binding looks for it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
SOURCES = ["pa_host.cpp", "pa_api.cpp", "pa_decode.hip", "pa_tiles.hip", "pa_append.hip", "pa_noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wextra",
    "-Werror",
    "-Wno-unused-parameter",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unknown-warning-option",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, defines: tuple = (), out: str = LIB) -> str:
    """Compile every source and link libpa.so at `out`; `defines` are extra
    -D options (tuning constants such as PA_TAIL_PERMILLE=150)."""
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC] + [f"-D{d}" for d in defines]
    with tempfile.TemporaryDirectory(prefix="pa_build_") as tmp:

        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [hipcc(), *HIPCC_FLAGS, *inc, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            # the host pass does not know the packed-fp32 feature name; that
            # note is expected and harmless
            noise = "is not a recognized feature for this target"
            msg = "\n".join(x for x in (r.stdout + r.stderr).splitlines() if noise not in x)
            if r.returncode != 0:
                raise RuntimeError(f"compiling {src} failed:\n{msg}")
            if msg.strip() and verbose:
                print(msg)
            return obj

        # one compiler process per source, at most four at a time
        with ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as pool:
            objs = list(pool.map(compile_one, SOURCES))
        tmp_lib = os.path.join(tmp, "libpa.so")
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"linking libpa.so failed:\n{r.stdout}{r.stderr}")
        os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
        shutil.move(tmp_lib, out)
    return out


HOST_SOURCES = ["pa_host.cpp", "pa_api.cpp", "pa_host_stub.cpp"]


def build_host_sanitized(out: str) -> str:
    """The host code alone (validation, planning, prefix detection; the
    launches replaced by stand-ins that report no device), compiled by g++
    with AddressSanitizer and UndefinedBehaviorSanitizer: a CPU-only library
    with libpa's C ABI for the ABI and host-planner tests.  Load it with the
    ASan runtime preloaded (tests/test_host_sanitized.py does)."""
    gxx = shutil.which("g++")
    if not gxx:
        raise RuntimeError("g++ not found")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-Wall", "-Wextra", "-Werror",
           "-Wno-unused-parameter", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, f) for f in HOST_SOURCES], "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build of the host code failed:\n{r.stdout}{r.stderr}")
    return out


PROBE_SRC = os.path.join(HERE, "probe", "hbm_probe.hip")
PROBE_LIB = os.path.join(HERE, "libpa_probe.so")


def build_probe(out: str = PROBE_LIB) -> str:
    """The HBM load-path probe (a measurement aid that bench.py --hbm-probe
    runs; not part of libpa)."""
    with tempfile.TemporaryDirectory(prefix="pa_probe_") as tmp:
        tmp_lib = os.path.join(tmp, "libpa_probe.so")
        cmd = [hipcc(), *HIPCC_FLAGS, "-shared", PROBE_SRC, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            noise = "is not a recognized feature for this target"
            msg = "\n".join(x for x in (r.stdout + r.stderr).splitlines() if noise not in x)
            raise RuntimeError(f"compiling the HBM probe failed:\n{msg}")
        shutil.move(tmp_lib, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe())

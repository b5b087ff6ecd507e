"""The host side of the C ABI under AddressSanitizer.

Builds libisd with AddressSanitizer on the host code only (the device code
is compiled as usual; no kernel runs here) and runs test_abi.py against it
in a child process that preloads the sanitizer runtime: every argument check
of every entry point, the shape and workspace arithmetic, the error text of
isd_last_error and the tuning setters then run with their memory accesses
checked.  Leak checking is off (the interpreter itself keeps allocations to
exit).  Skipped when hipcc or the runtime is not installed.
"""

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_verification_amd", "csrc")
SOURCES = ["isd_step.hip", "isd_trunc.hip", "isd_fused.hip", "isd_lm_head.hip", "isd_decode.hip",
           "isd_probe.hip", "isd_api.hip"]
# host-only instrumentation: each sanitizer flag applies to the host pass
HOST_ASAN = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _build(out_dir):
    hipcc = _hipcc()
    common = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
              "-I", CSRC] + HOST_ASAN

    def compile_one(src):
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        r = subprocess.run(common + ["-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    lib = os.path.join(out_dir, "libisd_asan.so")
    r = subprocess.run(common + ["-shared", "-o", lib] + objs, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return lib


def test_abi_checks_under_address_sanitizer(tmp_path):
    runtime = _runtime()
    if runtime is None or _hipcc() is None:
        pytest.skip("hipcc or the AddressSanitizer runtime is not installed")
    lib = _build(str(tmp_path))
    env = dict(os.environ, ISD_TEST_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout

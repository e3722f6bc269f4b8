"""Host-side memory checking of the C ABI: the library's host part (argument
validation, scale sizing, dispatch, launch set-up in csrc/api.cpp) rebuilt
with AddressSanitizer, linked with the unchanged device objects, and the ABI
tests (every rejection path, the binding's checks) run against it in a child
process with the sanitizer runtime preloaded.  Host code only: the device code
is not instrumented, and nothing here launches a kernel."""
import glob
import os
import subprocess
import sys

import pytest

from conftest import ROOT

BUILD = os.path.join(ROOT, "_build")
OBJS = [os.path.join(BUILD, n) for n in ("gemm.o", "quant.o", "probe.o")]
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

CSRC = os.path.join(ROOT, "column_scaled_gemm_amd", "csrc")


def _objects_current():
    """Every device object exists and is newer than every kernel source and
    header (a stale object could lack a symbol the current api.cpp needs)."""
    if not all(os.path.exists(o) for o in OBJS):
        return False
    newest_src = max(os.path.getmtime(p) for p in glob.glob(os.path.join(CSRC, "*"))
                     if p.endswith((".hip", ".h")))
    return min(os.path.getmtime(o) for o in OBJS) >= newest_src


pytestmark = pytest.mark.skipif(
    not _objects_current() or not RUNTIME,
    reason="device objects missing or older than the sources (build first), "
           "or the sanitizer runtime missing")


def _hipcc():
    from column_scaled_gemm_amd import build
    return build._hipcc()


def test_abi_rejection_paths_are_clean_under_address_sanitizer(tmp_path):
    obj = str(tmp_path / "api_asan.o")
    lib = str(tmp_path / "libfp8sm_asan.so")
    host = ["-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer", "-ffp-contract=off",
            "-I", os.path.join(ROOT, "include"), "-I", BUILD, "-D__HIP_PLATFORM_AMD__",
            "-I", "/opt/rocm/include"]
    r = subprocess.run([_hipcc()] + host + ["-Xarch_host", "-fsanitize=address", "-x", "c++", "-c",
                       os.path.join(ROOT, "column_scaled_gemm_amd", "csrc", "api.cpp"), "-o", obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan",
                        "-Xarch_host", "-fsanitize=address", "-o", lib] + OBJS + [obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    runner = (
        "import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "from column_scaled_gemm_amd import fp8sm\n"
        "fp8sm.LIB_PATH = %r\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider', %r]))\n"
    ) % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_abi.py"))
    env = dict(os.environ, LD_PRELOAD=RUNTIME[-1],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([sys.executable, "-c", runner], capture_output=True, text=True, env=env,
                       cwd=str(tmp_path), timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out

"""Build libfp8sm.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m column_scaled_gemm_amd.build   (or __graft_entry__.build()).
Always recompiles; objects go to _build/, the library next to this file.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfp8sm.so")

SOURCES = ["quant.hip", "gemm.hip", "probe.hip", "api.cpp"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
    "-I", BUILD,          # silu_tables.inc, generated below
]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src, obj, verbose):
    cmd = [_hipcc()] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc()] + [f for f in FLAGS if f != "--offload-arch=gfx950"] + \
            ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
             "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def _gen_silu_tables():
    """Compile and run the host generator of the constant SiLU tables."""
    exe = os.path.join(BUILD, "gen_silu_tables")
    cmd = [shutil.which("g++") or "g++", "-std=c++17", "-O2", "-ffp-contract=off",
           "-fno-fast-math", os.path.join(CSRC, "gen_silu_tables.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gen_silu_tables build failed:\n" + r.stdout + r.stderr)
    r = subprocess.run([exe], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gen_silu_tables failed:\n" + r.stderr)
    with open(os.path.join(BUILD, "silu_tables.inc"), "w") as f:
        f.write(r.stdout)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    _gen_silu_tables()
    objs = [os.path.join(BUILD, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda p: _compile(p[0], p[1], verbose), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

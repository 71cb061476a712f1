"""Build libpa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m paged_kv_cache_47_amd.build [--debug]

Every source under ``csrc/`` is compiled to an object (in parallel) and
linked into ``paged_kv_cache_47_amd/libpa.so`` (``--debug``: into
``libpa_debug.so``, built with ``PA_DEBUG=1``: every write, attention and
copy first checks its device metadata and refuses a call that breaks a
precondition): ``.hip`` files (kernels and
the device-side C ABI) with hipcc, ``.cpp`` files (host bookkeeping, no GPU
code) with the host C++ compiler.  Packed-fp32 instructions are disabled for
every HIP compile; there is no fast-math (the int8 write relies on IEEE fp32
division).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpa.so")
LIB_DEBUG = os.path.join(HERE, "libpa_debug.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    # a lambda parameter that shadows a local of the kernel around it has sent
    # a load to the wrong address: refuse such shadowing outright
    "-Werror=shadow-all",
]


# Per-file additions.  The MFMA kernel never sees a NaN score (hidden keys
# are -inf, rows past a sequence are read from its last real row), so its
# maxima need no NaN-quieting canonicalisation: 16 fewer VALU per 64-key step.
FILE_FLAGS = {"prefill.hip": ["-fno-honor-nans"]}


CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def cxx() -> str:
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand and shutil.which(cand):
            return cand
    raise RuntimeError("no host C++ compiler found")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature and says so; drop that line only
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(x for x in (r.stdout + r.stderr).splitlines() if noise not in x).strip()
    return msg


def build(debug: bool = False, verbose: bool = False) -> str:
    cc = hipcc()
    out_dir = os.path.join(BUILD, "debug") if debug else BUILD
    os.makedirs(out_dir, exist_ok=True)
    extra = ["-DPA_DEBUG=1"] if debug else []
    objs = []

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        if src.endswith(".cpp"):
            cmd = [cxx(), *CXX_FLAGS, *extra]
        else:
            cmd = [cc, *HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra]
        msg = _run([*cmd, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj])
        if verbose and msg:
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(compile_one, sources()))
    lib = LIB_DEBUG if debug else LIB
    tmp = lib + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    path = build(debug="--debug" in sys.argv, verbose=True)
    print(path)

"""Build libmtp.so (gfx950) in-tree with hipcc.

    python -m mtp_speculative_draft_amd.build

Each source compiles to an object under ``_build/`` in parallel, then one
shared library is linked next to this file.  The library is always rebuilt
when ``build()`` is called.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmtp.so")
SOURCES = ["gemv.hip", "attn.hip", "moe.hip", "api.cpp", "noalloc.hip"]
# measurement support for bench.py (a plain read stream), a library of its own
BENCH_LIB_PATH = os.path.join(HERE, "libmtp_bench.so")
BENCH_SOURCES = ["bench_stream.hip"]
ARCH = "gfx950"

# Packed-FP32 VALU forms are kept out of the generated code on purpose.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    _build_lib(SOURCES, LIB_PATH, verbose)
    _build_lib(BENCH_SOURCES, BENCH_LIB_PATH, verbose)
    return LIB_PATH


def _build_lib(sources, lib_path: str, verbose: bool) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in sources:
        obj = os.path.join(BUILD_DIR, src.replace(".", "_") + ".o")
        objs.append(obj)
        cmd = [cc, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l)
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = lib_path + ".tmp%d" % os.getpid()
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

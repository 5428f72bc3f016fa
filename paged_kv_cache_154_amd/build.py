"""Build the HIP shared library ``libpagedkv.so`` in-tree for gfx950.

    python -m paged_kv_cache_154_amd.build

Every call compiles from source (hipcc cross-compiles; no GPU is needed).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpagedkv.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["api.cpp", "decode.hip", "cache_ops.hip", "stream_read.hip", "shared_prefix.hip", "noalloc.hip"]

# Packed fp32 instructions are turned off for all device code.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libpagedkv.so")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, link libpagedkv.so."""
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="pagedkv_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [cc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                           stderr=subprocess.STDOUT, text=True), src))
            objs.append(obj)
        errors = []
        for pr, src in procs:
            out, _ = pr.communicate()
            msgs = [ln for ln in out.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in ln]
            if pr.returncode != 0:
                errors.append(f"{src}:\n" + "\n".join(msgs))
            elif verbose and msgs:
                print("\n".join(msgs), flush=True)
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n\n".join(errors))
        out_tmp = LIB_PATH + ".tmp"
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out_tmp], verbose)
        os.replace(out_tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

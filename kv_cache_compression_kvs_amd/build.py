"""Build libkvs.so in-tree: hipcc for the gfx950 kernels, g++ for the host ABI layer.

    python -m kv_cache_compression_kvs_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from typing import List

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvs.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["score_bf16.hip", "score_f32.hip", "select.hip", "copy.hip", "decode.hip",
               "calib.hip", "cluster.hip", "trace.hip", "scratch.hip"]
HOST_SOURCES = ["kvs_api.cpp"]

# Packed fp32 instructions (v_pk_fma_f32 and friends) are kept out of every
# device build; the host pass of hipcc warns that it does not know the
# feature, which is harmless.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd: List[str], verbose: bool) -> subprocess.Popen:
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _wait(procs):
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        useful = "\n".join(line for line in out.splitlines()
                           if "packed-fp32-ops" not in line)
        if p.returncode != 0:
            failed.append((cmd, useful))
        elif useful.strip():
            print(useful, file=sys.stderr)
    if failed:
        msg = "\n\n".join(" ".join(c) + "\n" + o for c, o in failed)
        raise RuntimeError("libkvs build failed:\n" + msg)


def build(verbose: bool = False) -> str:
    """Compile every source and link libkvs.so; always rebuilds.  Returns the path."""
    os.makedirs(BUILD, exist_ok=True)
    objs, procs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmd = [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, _run(cmd, verbose)))
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmd = ["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, _run(cmd, verbose)))
        objs.append(obj)
    _wait(procs)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    _wait([(cmd, _run(cmd, verbose))])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

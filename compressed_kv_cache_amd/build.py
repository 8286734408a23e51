"""Compile libdkv_attn.so for gfx950 with hipcc (in-tree, next to this file).

Each translation unit is compiled to an object of its own, in parallel, and the
objects are linked into one shared library."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SRCS = [os.path.join(CSRC, n) for n in ("dkv_attn.hip", "dkv_stream.hip", "dkv_seal.hip")]
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libdkv_attn.so")
OBJDIR = os.path.join(HERE, "_build")

# Packed fp32 VALU ops are switched off for every HIP translation unit.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-result"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return cmd


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    objs = [os.path.join(OBJDIR, os.path.basename(s).replace(".hip", ".o")) for s in SRCS]
    cmds = [[cc] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", s, "-o", o] for s, o in zip(SRCS, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for cmd in ex.map(_run, cmds):
            if verbose:
                print(" ".join(cmd))
    tmp = OUT + ".tmp"
    link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    _run(link)
    if verbose:
        print(" ".join(link))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))

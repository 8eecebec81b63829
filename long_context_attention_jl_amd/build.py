"""Build libjetlong.so (HIP, gfx950) in-tree with hipcc.

Each ``csrc/*.hip`` file is compiled to an object in parallel, then linked
into ``long_context_attention_jl_amd/libjetlong.so``.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libjetlong.so")
BUILD = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms stay disabled in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + list(extra) + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(msgs)))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(sys.argv[1:]))

"""Build libpagedattn.so for gfx950 with hipcc (in-tree, no JIT cache)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "pagedattn.hip")
DEPS = [SRC, os.path.join(PKG, "csrc", "pa_kernels.h"), os.path.join(PKG, "csrc", "pa_prefill.h"),
        os.path.join(PKG, "csrc", "pa_stream.h"),
        os.path.join(ROOT, "include", "pagedattn.h")]
SO = os.path.join(PKG, "libpagedattn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # packed-fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def command(out: str = SO):
    return [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), SRC, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = SO + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libpagedattn.so")
    os.replace(tmp, SO)
    return SO


def is_stale() -> bool:
    if not os.path.exists(SO):
        return True
    t = os.path.getmtime(SO)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))

"""Compiles the HIP sources of the library into libentmaxkv.so (gfx950)."""
from __future__ import annotations

import glob
import os
import subprocess
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libentmaxkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 arithmetic in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG_DIR, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every .hip source into one shared library; returns its path.
    The library is written next to this file and replaced atomically."""
    fd, tmp = tempfile.mkstemp(suffix=".so.tmp", dir=PKG_DIR)
    os.close(fd)
    cmd = [HIPCC, *FLAGS, "-o", tmp, *sources()]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
        if verbose:
            print(" ".join(cmd))
        os.replace(tmp, LIB_PATH)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))

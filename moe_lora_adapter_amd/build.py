"""Build libmoelora.so (the HIP kernels and the C ABI) for gfx950, in-tree."""

from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoelora.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result", "-fvisibility=hidden",
    # packed fp32 instructions stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out: str = LIB, extra: tuple = (), verbose: bool = False) -> str:
    """Compile every HIP source into one shared library; return its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *extra,
           *sources(), "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + msg)
    if verbose and msg.strip():
        print(msg)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libgpulz.so in-tree with hipcc for gfx950.

Run ``python -m chunked_lzss_coder_amd.build``.  Always recompiles."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed FP32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-fvisibility=hidden",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(_HERE, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    out = os.path.join(_HERE, "libgpulz.so")
    tmp = f"{out}.{os.getpid()}.tmp"  # one per process: concurrent builds do not collide
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(_ROOT, "include"), "-I", os.path.join(_HERE, "csrc"),
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build liblact.so (gfx950 only) in-tree with hipcc.

    python -m test_layers_amd.build
"""
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "lact.hip")
OUT = os.path.join(PKG, "liblact.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep hipcc from emitting packed fp32 ops (device pass; the host pass
    # warns that it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for c in [os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")]:
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblact)")


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           SRC, "-o", tmp]
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{err}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} in {time.time() - t:.1f}s")
        if err.strip():
            print(err)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

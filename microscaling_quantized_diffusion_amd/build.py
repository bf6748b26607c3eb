"""Build libmxq.so (HIP kernels + C-ABI host code) in-tree for gfx950.

    python -m microscaling_quantized_diffusion_amd.build

Every translation unit under csrc/ is compiled with hipcc for gfx950 only and
linked into ``microscaling_quantized_diffusion_amd/libmxq.so``.  Packed-FP32
VALU instructions are disabled for the device code.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(REPO_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libmxq.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(REPO_DIR, 'include')}",
]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every csrc/*.hip for gfx950 and link libmxq.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    srcs = sources()
    pending = list(srcs)
    running = []

    while pending or running:
        while pending and len(running) < jobs:
            src = pending.pop(0)
            obj = os.path.join(BUILD_DIR, os.path.basename(src).replace(".hip", ".o"))
            objs.append(obj)
            cmd = [hipcc, *HIPCC_FLAGS, "-c", src, "-o", obj]
            p = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
            running.append((p, src, p.stdout))
        if running:
            p, src, log = running[0]
            out = log.read()
            p.wait()
            running.pop(0)
            if p.returncode != 0:
                for q, _, _ in running:
                    q.wait()
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
            # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that line
            msgs = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if verbose and msgs:
                print("\n".join(msgs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)

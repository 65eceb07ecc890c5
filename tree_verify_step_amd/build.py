"""Build the gfx950 HIP library libmedusa_verify.so in-tree with hipcc.

Every source under csrc/ is compiled as HIP for gfx950 (one code path) and
linked into tree_verify_step_amd/libmedusa_verify.so.  Packed-FP32 VALU
instructions are disabled (-packed-fp32-ops) for the device pass.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libmedusa_verify.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


# Per-source extra flags.  The GEMM keeps its MFMA accumulators in VGPRs:
# with AGPR accumulators the register allocator rotates them through copies
# that wait on each MFMA result.
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, obj: str) -> str:
    cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           *EXTRA.get(os.path.basename(src), []),
           "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the device-only feature name: drop that noise
    noise = "'-packed-fp32-ops' is not a recognized feature"
    return "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for src, warn in zip(srcs, ex.map(_compile, srcs, objs)):
            if warn.strip() and verbose:
                print(f"[build] {os.path.basename(src)}:\n{warn}", file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"[build] wrote {OUT}", file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build()

"""Build libnabla.so (HIP, gfx950) in-tree with hipcc.

    python -m block_sparse_attention_flatten_amd.build
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libnabla.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for all device code (hipcc would
# otherwise emit them from plain float code).
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
_NOISE = "is not a recognized feature for this target"

# Per-source extras.  The pipelined attention kernel takes row maxima of
# matrix-core results, which are never NaN for finite inputs; without NaN
# semantics the compiler drops the canonicalising moves it would otherwise
# put in front of every v_max.
FILE_FLAGS = {"attn_fwd_vt.hip": ["-fno-honor-nans"]}


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libnabla")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if _NOISE not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)


def build_library(out: str = LIB, verbose: bool = False) -> str:
    """Compile every HIP source (in parallel) and link one shared library."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include")]
    jobs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        extra = FILE_FLAGS.get(os.path.basename(src), [])
        jobs.append((obj, [cc, *HIP_FLAGS, *extra, *inc, "-c", src, "-o", obj]))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda j: _run(j[1], verbose), jobs))
    tmp = out + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in jobs]],
         verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))

"""Build libsplitkv.so for gfx950 in-tree with hipcc.

Usage: python -m split_kv_amd.build [-v]

Every HIP source is compiled for gfx950 only, with packed-fp32 code
generation turned off, then linked into ``split_kv_amd/libsplitkv.so``.
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
LIB = os.path.join(PKG, "libsplitkv.so")
BUILD_DIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _revision() -> str:
    try:
        out = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"],
                             capture_output=True, text=True, timeout=10)
        rev = out.stdout.strip() or "unknown"
        dirty = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--", "split_kv_amd/csrc",
                                "include"], capture_output=True, text=True, timeout=10).stdout.strip()
        return rev + ("-dirty" if dirty else "")
    except (OSError, subprocess.SubprocessError):
        return "unknown"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


# Per-source code-generation options.  The grouped-query and short-range MLA
# kernels rescale their MFMA accumulators with vector ALU code; keeping them
# in VGPRs (instead of the accumulation registers) avoids copying them across
# on every group or tile.  The
# grouped-query and combine kernels take their first fourteen argument dwords
# preloaded into scalar registers at wave launch, so their first memory access
# does not wait for an argument load.
PER_FILE = {
    "gqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true", "-mllvm", "-amdgpu-kernarg-preload-count=14"],
    "combine.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=14"],
    "mla_short.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
    "mla_short_q8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
}


def _compile(src: str, rev: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    extra = PER_FILE.get(os.path.basename(src), [])
    cmd = [HIPCC, *FLAGS, *extra, f'-DSPLITKV_REVISION="{rev}"', "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    noisy = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noisy:
        print("\n".join(noisy), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    rev = _revision()
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, rev, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} ({rev})", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)

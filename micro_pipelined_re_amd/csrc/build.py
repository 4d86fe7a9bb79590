"""Builds libgpipe_cell.so (gfx950) from the HIP sources next to this file.

    python -m micro_pipelined_re_amd.csrc.build

Objects go to _build/ at the repository root; the library is written into the
package directory so it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgpipe_cell.so")
SOURCES = ["gemm.hip", "gemm_fwd.hip", "gemm_dgrad.hip", "gemm_wgrad.hip", "gemm_attn.hip",
           "gemm_f32.hip", "rowops.hip", "convops.hip", "conv_cell.hip", "attn.hip",
           "gpipe_api.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 instructions are emitted (host pass warns that it does not know it)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, out_dir: str) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noisy = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noisy:
        sys.stderr.write("\n".join(noisy) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    # native driver of the C-ABI step (for profiling without an interpreter)
    exe = os.path.join(PKG, "cell_bench")
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", exe + ".tmp", os.path.join(HERE, "cell_bench.cpp"),
           f"-L{PKG}", "-lgpipe_cell", "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"cell_bench build failed:\n{r.stderr}")
    os.replace(exe + ".tmp", exe)
    if verbose:
        print(f"built {LIB} and {exe}")
    return LIB


if __name__ == "__main__":
    build()

"""Build libflashattn.so (gfx950) in-tree with hipcc.

``build()`` always recompiles every source.  Objects go to ``_build/`` at the
repository root; the shared library lands next to this file, where the
Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libflashattn.so")
OBJ = os.path.join(ROOT, "_build")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd2.hip", "fa_fwd_f32.hip", "fa_bwd.hip", "fa_decode.hip", "fa_noalloc.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm 7.x required to build libflashattn.so)")


def _spills(remarks: str):
    """Kernels the compiler reports with register spills (resource-usage remarks)."""
    bad, name = [], None
    for line in remarks.splitlines():
        if "remark:" not in line:
            continue
        txt = line.split("remark:", 1)[1].strip()
        if txt.startswith("Function Name:"):
            name = txt.split(":", 1)[1].strip()
        elif txt.startswith(("VGPRs Spill:", "SGPRs Spill:")):
            n = int(txt.split(":", 1)[1].split()[0])
            if n and name:
                bad.append(f"{name} ({txt.split(' [')[0]})")
    return bad


def _compile(src: str, extra) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-Rpass-analysis=kernel-resource-usage",
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # The backward kernels issue matrix products and DMA through inline asm
    # whose hazards the compiler does not see; spill code (register copies
    # and scratch memory traffic inside the loops) would break the
    # assumptions those asm statements rely on.  Refuse such a build.
    bad = _spills(r.stderr)
    if bad:
        raise RuntimeError(f"{src}: register spills in " + ", ".join(bad))
    return obj


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)

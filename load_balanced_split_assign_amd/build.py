"""Build liblbsa.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

``python -m load_balanced_split_assign_amd.build`` compiles every translation
unit under ``csrc/`` and links ``load_balanced_split_assign_amd/liblbsa.so``
in-tree.  hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "lbsa")
LIB = os.path.join(HERE, "liblbsa.so")
SOURCES = ["lbsa_assign.hip", "lbsa_attention.hip", "lbsa_prefill.hip", "lbsa_prologue.hip", "lbsa_router.hip",
           "lbsa_api.hip"]
ARCH = os.environ.get("LBSA_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed FP32 math is kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
]


# per-source flags: the prefill and router kernels keep their MFMA
# accumulators in VGPRs.  Prefill: the softmax rescale touches them with VALU
# instructions, which cannot read AGPRs.  Router: with AGPR accumulators
# carried around the k loop, the allocator reshuffles them with accvgpr moves
# on every iteration.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# the decode kernels take the arguments of their first dependent loads (the map
# pointer and the shape words) as leading scalar parameters, which gfx950
# preloads into SGPRs before the first instruction: the map loads go out
# without waiting for a kernel-argument load
_PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=8"]
EXTRA = {"lbsa_prefill.hip": _VGPR_FORM, "lbsa_router.hip": _VGPR_FORM, "lbsa_attention.hip": _PRELOAD,
         "lbsa_assign.hip": _PRELOAD}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def build(verbose: bool = False) -> str:
    """Compile all sources and link liblbsa.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

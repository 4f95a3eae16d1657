"""Build libgdn.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m gated_deltanet_recurrent_delta_amd.build [--clean] [-j N]

Objects go to _build/ at the repository root; the shared library is written
next to this file so the binding finds it.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")

SOURCES = ["gdn_api.hip", "gdn_backward.hip", "gdn_backward_chunk.hip", "gdn_decode.hip", "gdn_gated.hip", "gdn_gated_chunk.hip", "gdn_noalloc.hip",
           "gdn_prefill.hip", "gdn_select.hip", "gdn_truncate.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep packed-fp32 VALU ops out of device code (a hipcc device flag; the
    # host pass warns that it does not know it)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in architectural VGPRs: otherwise values loaded
    # from memory and later used as accumulators are copied into AGPRs right
    # at the load, which forces a wait on the load (and on every vector
    # memory operation issued before it, prefetches included)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs)
    return obj


def build(verbose: bool = False, jobs: int = 4, clean: bool = False) -> str:
    """Compile every source for gfx950 and link libgdn.so; returns its path."""
    if clean and os.path.isdir(BUILD):
        shutil.rmtree(BUILD)
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--clean", action="store_true")
    ap.add_argument("-j", "--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.verbose, a.jobs, a.clean))
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Host-sanitized build of libgdn for tests on the CPU.

    python -m gated_deltanet_recurrent_delta_amd.build_hostsan

The host code of the library (argument checks, workspace sizing, dispatch
and the host DRRQR channel selector; gdn_api.hip, gdn_noalloc.hip and
gdn_select.hip) is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only; the device code is not
instrumented.  The other objects come from the regular build in _build/.
The result, _build/hostsan/libgdn.so, is loaded by a Python process started
with the sanitizer runtime preloaded (see runtime()) and GDN_LIB_PATH
pointing at it.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

from gated_deltanet_recurrent_delta_amd import build as _b

HOST_SOURCES = ["gdn_api.hip", "gdn_noalloc.hip", "gdn_select.hip"]
OUT = os.path.join(_b.BUILD, "hostsan")
LIB = os.path.join(OUT, "libgdn.so")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def runtime() -> str | None:
    """Path of clang's shared AddressSanitizer runtime, or None."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in _b.SOURCES:
        if src in HOST_SOURCES:
            obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
            cmd = [_b.HIPCC, *_b.FLAGS, *SAN, "-c", os.path.join(_b.CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        else:
            obj = os.path.join(_b.BUILD, os.path.splitext(src)[0] + ".o")
            if not os.path.exists(obj):
                _b._compile(src, False)
        objs.append(obj)
    cmd = [_b.HIPCC, f"--offload-arch={_b.ARCH}", "-shared", "-fPIC", *objs,
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-shared-libasan", "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)

"""Build libprox.so in-tree with hipcc for gfx950 (CDNA4, MI355X).

Each translation unit is compiled on its own (in parallel), then linked into
one shared library next to this file."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libprox.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["prox_kernels.hip", "prox_fused.hip", "prox_sgemv.hip", "prox_api.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops off (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Per-source additions.  Every atomic of the persistent kernel is issued by a
# single lane, where the atomic optimizer's wave-wide scan only adds work.
FILE_FLAGS = {"prox_fused.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def build(verbose: bool = False, incremental: bool = False, extra_flags=()) -> str:
    """Compile every source (incremental: only those whose object is older
    than the source or a header) and link libprox.so.  extra_flags go on
    every compile and on the link line (the CPU sanitizer run passes
    -Xarch_host -fsanitize=... here)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    headers = [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")]
    headers.append(os.path.join(os.path.dirname(HERE), "include", "prox.h"))
    newest_hdr = max(os.path.getmtime(h) for h in headers)

    def compile_one(src):
        obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        if incremental and os.path.exists(obj):
            t = os.path.getmtime(obj)
            if t > os.path.getmtime(os.path.join(CSRC, src)) and t > newest_hdr:
                return obj
        cmd = [hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), *extra_flags, "-c", "-o", obj,
               os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.check_call(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *extra_flags,
                           "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    # python build.py [-i] [--sanitize]: --sanitize builds the host code with
    # AddressSanitizer and UndefinedBehaviorSanitizer (device code untouched).
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"] if "--sanitize" in sys.argv else []
    print(build(verbose=True, incremental="-i" in sys.argv, extra_flags=san))

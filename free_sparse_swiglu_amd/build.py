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


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (incremental: only those whose object is older
    than the source or a header) and link libprox.so."""
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
        cmd = [hipcc, *HIPCC_FLAGS, "-c", "-o", obj, os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.check_call(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, incremental="-i" in sys.argv))

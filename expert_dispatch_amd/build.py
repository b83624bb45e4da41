"""Build libmoe.so (the HIP library behind include/moe.h) for gfx950.

    python -m expert_dispatch_amd.build [--debug]

Each source is compiled to an object in ``_build/`` (in parallel), then
linked in-tree as ``expert_dispatch_amd/libmoe.so``. Packed fp32 VALU
instructions are switched off for every device compile.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["api.hip", "route.hip", "permute.hip", "grouped_ffn.hip", "grouped_bwd.hip",
           "combine.hip", "ceiling.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_LIB = "/opt/rocm/lib"

CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


LIB_DEBUG = os.path.join(PKG, "libmoe_debug.so")


def build(verbose: bool = False, debug: bool = False) -> str:
    """Build libmoe.so, or with ``debug`` libmoe_debug.so: the same sources
    compiled with MOE_DEBUG, whose kernels record broken device-side
    preconditions for moe_debug_status (test-only)."""
    bdir = os.path.join(BUILD, "debug") if debug else BUILD
    out_lib = LIB_DEBUG if debug else LIB
    os.makedirs(bdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *CFLAGS, *(["-DMOE_DEBUG"] if debug else []), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 feature; that note is harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or p.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = out_lib + ".tmp"
    # -Bsymbolic: the library's own calls bind inside it, so the release and
    # the debug library can be open in one process side by side
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-Bsymbolic", *objs,
                    "-L", ROCM_LIB, "-Wl,-rpath," + ROCM_LIB, "-lrocprofiler-sdk-roctx",
                    "-o", tmp], check=True)
    os.replace(tmp, out_lib)
    return out_lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv))

"""Build libnormrope.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m rmsnorm_layernorm_fwd_amd.build [--incremental]

Each .hip file under csrc/ is compiled to an object in parallel, then linked
into rmsnorm_layernorm_fwd_amd/libnormrope.so.  Packed-fp32 instruction
selection is switched off for the device code (-packed-fp32-ops); the host
pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnormrope.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _compile(src: str, newest_header: float = None) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if newest_header is not None and os.path.exists(obj):
        deps = [os.path.getmtime(src), newest_header]
        with open(src) as fh:
            if "normrope.h" in fh.read():
                deps += [os.path.getmtime(h) for h in glob.glob(os.path.join(HERE, "..", "include", "*.h"))]
        if os.path.getmtime(obj) > max(deps):
            return obj
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compiles every source (incremental: only those older than their
    object, headers included) and links the library."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    headers = glob.glob(os.path.join(CSRC, "*.hpp"))
    newest = max(os.path.getmtime(h) for h in headers) if incremental else None
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, newest), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)

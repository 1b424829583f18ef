"""Build libnucleus.so in-tree with hipcc for gfx950.

    python -m nucleus_sampling_amd.build [--stamps]

--stamps builds libnucleus_stamps.so instead: the same library with the
one-workgroup-per-row kernel's phase clocks compiled in (NUCLEUS_PHASE_STAMPS,
read with `python -m nucleus_sampling_amd.phase_stamps`).

Every HIP source is compiled with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass warns that
it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnucleus.so")
LIB_STAMPS = os.path.join(HERE, "libnucleus_stamps.so")
SOURCES = [os.path.join(CSRC, "nucleus.hip")]
OBJDIR = os.path.join(ROOT, "_build")
EXTRA = {}  # per-source extra hipcc flags

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False, only=None, stamps: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the
    library.  ``only`` (a list of source basenames) recompiles just those and
    relinks with the other objects as they are."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(OBJDIR, "stamps") if stamps else OBJDIR
    out = LIB_STAMPS if stamps else LIB
    defines = ["-DNUCLEUS_PHASE_STAMPS"] if stamps else []
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        if only is not None and os.path.basename(src) not in only and os.path.exists(obj):
            continue
        cmd = [hipcc, *HIPCC_FLAGS, *defines, *EXTRA.get(os.path.basename(src), []), "-c", "-o", obj + ".tmp", src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), obj))
    for pr, obj in procs:
        if pr.wait() != 0:
            raise subprocess.CalledProcessError(pr.returncode, f"hipcc -c for {obj}")
        os.replace(obj + ".tmp", obj)
    tmp = out + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    only = [a for a in sys.argv[1:] if a.endswith(".hip")] or None
    build(verbose="-v" in sys.argv, only=only, stamps="--stamps" in sys.argv)

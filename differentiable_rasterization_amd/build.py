"""Build libgsraster.so (hand-written HIP for gfx950) in-tree with hipcc.

Flags:
  -ffp-contract=off   the projection's key path must be bit-reproducible and
                      the compositing forward/backward must replay the same
                      decisions; fused multiply-adds are written explicitly.
  -munsafe-fp-atomics fp32 atomicAdd lowers to the hardware global atomic.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed fp32 instructions are emitted.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgsraster.so")
# sha256 of the sources and flags a library was built from, written beside it
HASH_FILE = LIB + ".srchash"
SOURCES = ["project.hip", "binsort.hip", "raster.hip", "densify.hip", "train.hip",
           "api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-munsafe-fp-atomics", "-fvisibility=hidden",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
            "-Wall", "-Wno-unused-result"]


def source_hash() -> str:
    """sha256 over the HIP sources, their headers, the C ABI header and the
    compile flags."""
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    for f in files:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "include", "gsraster.h"), "rb") as fh:
        h.update(fh.read())
    h.update(" ".join(flags()).replace(ROOT, "").encode())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + flags() + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libgsraster.so")
    os.replace(tmp, LIB)
    with open(HASH_FILE, "w") as fh:
        fh.write(source_hash() + "\n")
    return LIB


def dump_isa(out_dir: str) -> None:
    """Write the gfx950 assembly of every source (for inspection of our own
    kernels' instruction counts)."""
    os.makedirs(out_dir, exist_ok=True)
    for s in SOURCES:
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-ffp-contract=off",
               "-munsafe-fp-atomics", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "--cuda-device-only", "-S",
               os.path.join(CSRC, s), "-o", os.path.join(out_dir, s.replace(".hip", ".s"))]
        subprocess.run(cmd, check=True)


if __name__ == "__main__":
    print(build(verbose=True))

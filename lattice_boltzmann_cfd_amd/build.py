"""Compile liblbm_hip.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m lattice_boltzmann_cfd_amd.build``; ``__graft_entry__.build()``
calls :func:`build`.  The library is written next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblbm_hip.so")
SOURCES = [os.path.join(CSRC, "lbm_kernels.hip"), os.path.join(CSRC, "lbm_api.cpp")]
HEADERS = [os.path.join(ROOT, "include", "lbm.h"), os.path.join(CSRC, "lbm_lattice.hpp"),
           os.path.join(CSRC, "lbm_internal.hpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def command(out=LIB, extra=()):
    return [
        HIPCC, "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 instructions stay off (they are not used by hand either)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # fuse a*b+c only inside one source expression: the same collision code
        # then rounds identically in every kernel that inlines it, whatever
        # branches surround it (in-place and two-buffer results agree bitwise)
        "-ffp-contract=on",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *extra, "-o", out, *SOURCES, "-lpthread",
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def up_to_date() -> bool:
    if not os.path.exists(LIB):
        return False
    t = os.path.getmtime(LIB)
    return all(os.path.getmtime(s) <= t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build step for the HIP library (libmk.so, gfx950) and the host-side input generator.

Compiles in-tree with hipcc so the built library travels with the source tree. Every HIP translation
unit is built with packed fp32 instructions disabled (they are emitted only from ordinary float code
otherwise, and some of their forms are not trusted on this hardware)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def build_lib(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, "mk_host.cpp"), os.path.join(CSRC, "mk_device.hip")]
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + HIP_FLAGS + ["-shared", "-x", "hip"] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmk.so")
    os.replace(tmp, LIB)
    return LIB


def build_all(verbose: bool = False) -> None:
    from persistent_megakernel_mk_amd import synth

    synth.build_host_lib(force=True)
    synth.build_gpu_lib()
    build_lib(verbose)


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    build_all(verbose=True)
    print("built", LIB)

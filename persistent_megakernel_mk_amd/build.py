"""Build step for the HIP library (libmk.so, gfx950) and the host-side input generator.

Compiles in-tree with hipcc so the built library travels with the source tree. The library has four
translation units (the host runtime and the three builds of the step kernel), compiled in parallel and
linked together. Every HIP translation unit is built with packed fp32 instructions disabled (they are
emitted only from ordinary float code otherwise, and some of their forms are not trusted on this
hardware)."""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OBJ_DIR = os.path.join(PKG, "_build")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
UNITS = ["mk_host.cpp", "mk_step.hip", "mk_step_nvfp4.hip", "mk_step_wide.hip"]


def build_lib(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    procs = []
    t0 = time.time()
    for u in UNITS:
        obj = os.path.join(OBJ_DIR, u + ".o")
        cmd = [HIPCC] + HIP_FLAGS + list(extra_flags) + ["-x", "hip", "-c", os.path.join(CSRC, u), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((u, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = False
    for u, _, p in procs:
        out, _ = p.communicate()
        if out.strip():
            sys.stderr.write(out)
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"hipcc failed on {u}\n")
        elif verbose:
            print(f"compiled {u} ({time.time() - t0:.0f} s)", flush=True)
    if failed:
        raise RuntimeError("hipcc failed building libmk.so")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for _, o, _ in procs] + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("linking libmk.so failed")
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

"""Build libserq.so in-tree with hipcc for gfx950.

    python w4a4_linear_layers_amd/build.py            # build (always recompiles)
    python w4a4_linear_layers_amd/build.py --asm DIR  # also dump device assembly

(Run as a script: importing the package would first load the library being
rebuilt.)

The library is one shared object: host C++ (calibration, C ABI) and the HIP
kernels, linked against the HIP runtime. Every floating-point step of the
quantizers is a single IEEE operation, so contraction into fused
multiply-adds is disabled (-ffp-contract=off); packed-fp32 VALU forms are
disabled as well.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libserq.so")
ARCH = os.environ.get("SERQ_OFFLOAD_ARCH", "gfx950")

SOURCES = ["serq_abi.cpp", "calibrate.cpp", "quant_act.hip", "serq_gemm.hip", "serq_mx.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
            "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument", "-Wno-unknown-warning-option",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False, asm_dir: str | None = None) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([cc] + common_flags() + lang + ["-c", path, "-o", obj])
        objs.append(obj)
        if asm_dir and src.endswith(".hip"):
            os.makedirs(asm_dir, exist_ok=True)
            out = os.path.join(asm_dir, os.path.splitext(src)[0] + ".s")
            cmds.append([cc] + common_flags() + lang + ["--cuda-device-only", "-S", path, "-o", out])
    # the translation units are independent: compile them side by side
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
    failed = [cmd for cmd, p in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="directory for device assembly listings")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(verbose=args.verbose, asm_dir=args.asm))
    return 0


if __name__ == "__main__":
    sys.exit(main())

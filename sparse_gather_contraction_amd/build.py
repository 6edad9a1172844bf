"""Build libdisco.so (hipcc, gfx950) in-tree.

    python -m sparse_gather_contraction_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdisco.so")
PROBE_LIB = os.path.join(PKG, "libdisco_probes.so")  # microbenchmarks of the device (measurement only)

SOURCES = ["plan.cpp", "plan_fused.cpp", "plan_tile.cpp", "kernels_tile.hip", "disco_api.hip", "kernels_gather.hip", "kernels_staged.hip", "kernels_fused.hip",
           "kernels_fused_mfma.hip", "kernels_gemm.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Device code is built with packed fp32 VALU ops disabled, and with unaligned memory access
# disabled: on gfx950 unaligned LDS reads stall the LDS pipeline (SQ_LDS_UNALIGNED_STALL), so
# reads at 2-byte alignment are kept as 2-byte reads instead of being merged into wide ones.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xclang", "-target-feature", "-Xclang", "-unaligned-access-mode",
         "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                     if "packed-fp32-ops" not in l and "unaligned-access-mode" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    undef = subprocess.run(["nm", "-D", "-C", "--undefined-only", tmp], stdout=subprocess.PIPE, text=True).stdout
    missing = [l.split()[-1] for l in undef.splitlines() if "disco::" in l or " disco_" in l]
    if missing:
        raise RuntimeError("libdisco.so has undefined symbols of its own: " + ", ".join(missing))
    os.replace(tmp, LIB)
    probe_obj = _compile("probes.hip")
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", probe_obj, "-o", tmp],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe link failed:\n" + r.stdout)
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

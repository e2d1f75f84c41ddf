"""Build libpkb.so (the attention library) and libpkb_peaks.so (on-device
ceilings used by the benchmark) in-tree for gfx950 (explicit hipcc / g++
invocations).

Usage: python paged_kv_block_amd/build.py [-j N]   (run by path: importing the
package loads the library this script builds)
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpkb.so")
PEAKS_LIB = os.path.join(HERE, "libpkb_peaks.so")

ARCH = os.environ.get("PKB_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include")]

HIP_SOURCES = ["attn_fwd.hip", "attn_ragged.hip", "decode_fwd.hip", "sage_fwd.hip", "qsa_fwd.hip",
               "api.cpp"]
# Per-source extra device flags.  The decode kernel fits in the 256 architectural
# VGPRs, so its MFMA operands and accumulators are kept there: VALU work on the
# accumulators (rescale, epilogue) then needs no AGPR <-> VGPR copies.
SOURCE_FLAGS = {"decode_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "attn_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "attn_ragged.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "qsa_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
CPP_SOURCES = ["host.cpp"]
PEAKS_SOURCES = ["peaks.hip"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def compile_one(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src in HIP_SOURCES or src in PEAKS_SOURCES:
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-x", "hip", "-c", path, "-o", obj,
               *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []),
               "-Wno-unused-command-line-argument"]
    else:
        cmd = ["g++", "-c", path, "-o", obj, *COMMON, "-Wall"]
    _run(cmd)
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = HIP_SOURCES + CPP_SOURCES + PEAKS_SOURCES
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = dict(zip(srcs, ex.map(compile_one, srcs)))
    for lib, group in ((LIB, HIP_SOURCES + CPP_SOURCES), (PEAKS_LIB, PEAKS_SOURCES)):
        tmp = lib + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[objs[x] for x in group],
              "-o", tmp])
        os.replace(tmp, lib)
        if verbose:
            print("built", lib)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=4)
    a = ap.parse_args(argv)
    build(a.j, verbose=True)


if __name__ == "__main__":
    sys.exit(main())

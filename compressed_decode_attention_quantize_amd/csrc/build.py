"""Builds libtq.so (the C-ABI library) for gfx950 with hipcc.

Usage: python compressed_decode_attention_quantize_amd/csrc/build.py [-j N]

Every call recompiles every source (no cache). Objects go to
compressed_decode_attention_quantize_amd/_build/, the library to
compressed_decode_attention_quantize_amd/libtq.so.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtq.so")

SOURCES = ["tq_host.cpp", "tq_api.cpp", "tq_quantize.hip", "tq_decode.hip", "tq_prefill.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-ffp-contract=off",
          "-Wall", "-Wno-unused-function"]
# Device code: gfx950 only; packed fp32 arithmetic is disabled on purpose.
DEVICE = ["-x", "hip", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMA accumulators in VGPRs: the online softmax rescales them with
          # VALU ops, which cannot read AGPRs
          "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON]
    if src.endswith(".hip"):
        cmd += DEVICE
    cmd += ["-c", os.path.join(HERE, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=min(4, os.cpu_count() or 1))
    a = ap.parse_args()
    try:
        build(a.j, verbose=True)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)

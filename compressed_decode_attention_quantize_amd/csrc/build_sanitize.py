"""CPU sanitizer build of the library's host code: tq_host.cpp and
tq_api.cpp (argument checks, work division, workspace layout, error
reporting) compiled by clang++ with AddressSanitizer and
UndefinedBehaviorSanitizer, linked with the device objects of the regular
build (csrc/build.py) into compressed_decode_attention_quantize_amd/_build_san/libtq.so.
No GPU code is instrumented.

Use: build_sanitized() returns the library path; load it through the binding
with TQ_LIBRARY=<path> and the ASan runtime preloaded
(LD_PRELOAD=asan_runtime(), ASAN_OPTIONS=detect_leaks=0: the Python
interpreter itself is not instrumented).
"""

from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
BUILD = os.path.join(PKG, "_build")
OUT = os.path.join(PKG, "_build_san")
ROCM = "/opt/rocm"
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
HOST_SOURCES = ["tq_host.cpp", "tq_api.cpp"]
DEVICE_OBJECTS = ["tq_quantize.o", "tq_decode.o", "tq_prefill.o"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    found = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not found:
        raise FileNotFoundError("no libclang_rt.asan-x86_64.so under the ROCm LLVM")
    return found[-1]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


def build_sanitized() -> str:
    missing = [o for o in DEVICE_OBJECTS if not os.path.exists(os.path.join(BUILD, o))]
    if missing:
        import build  # noqa: E402  (csrc/build.py, this directory)
        build.build()
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        _run([CLANGXX, "-std=c++17", "-fPIC", "-O1", "-g", "-fvisibility=hidden", *SAN,
              "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
              "-c", os.path.join(HERE, src), "-o", obj])
        objs.append(obj)
    lib = os.path.join(OUT, "libtq.so")
    _run([CLANGXX, "-shared", *SAN, "-shared-libasan", *objs, *[os.path.join(BUILD, o) for o in DEVICE_OBJECTS],
          "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-o", lib])
    return lib


if __name__ == "__main__":
    print(build_sanitized())

"""Build ``libnvfp4.so`` from the HIP sources in ``csrc/`` with hipcc for gfx950.

Every source is compiled with -ffp-contract=off (the quantizers must perform single IEEE fp32
operations), with packed-fp32 instructions disabled, and with hidden visibility, and linked
with a version script (csrc/exports.map): the library exports exactly the C ABI.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libnvfp4.so")
SOURCES = ["quantize.hip", "hadamard.hip", "gemm.hip", "gemm_mx.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    subprocess.run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], check=True)
    return obj


def build() -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                    "-Wl,--version-script=" + os.path.join(CSRC, "exports.map"), "-o", tmp, *objs],
                   check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())

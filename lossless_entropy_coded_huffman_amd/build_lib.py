"""Build libdfh.so in-tree for gfx950: the host half with g++, the HIP half
with hipcc, linked by hipcc.  ``python -m lossless_entropy_coded_huffman_amd.build_lib``
or ``__graft_entry__.build()`` run it."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(BUILD, "libdfh.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include")]
    host_o = os.path.join(BUILD, "dfh_host.o")
    dev_o = os.path.join(BUILD, "dfh_decode.o")
    _run(["g++", "-O3", "-std=c++17", "-fPIC", "-pthread", "-Wall", "-Wextra",
          "-D__HIP_PLATFORM_AMD__"] + inc + ["-c", os.path.join(CSRC, "dfh_host.cpp"), "-o", host_o])
    _run([os.path.join(ROCM, "bin", "hipcc")] + HIP_FLAGS + inc +
         ["-c", os.path.join(CSRC, "dfh_decode.hip"), "-o", dev_o])
    enc_o = os.path.join(BUILD, "dfh_encode.o")
    _run([os.path.join(ROCM, "bin", "hipcc")] + HIP_FLAGS + inc +
         ["-c", os.path.join(CSRC, "dfh_encode.hip"), "-o", enc_o])
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([os.path.join(ROCM, "bin", "hipcc"), "-shared", "-fPIC", "--offload-arch=" + ARCH,
          host_o, dev_o, enc_o, "-pthread", "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)

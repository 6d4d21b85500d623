"""Build the HIP library (libll.so, gfx950), the CPU-only recording variant (libll_fake.so),
its sanitizer-instrumented twin (libll_fake_san.so) and the plain-C consumer the C-ABI test
runs (tests/c_abi_stream) in-tree. Run `python -m windowed_attention_kv_amd.build`."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
HIP_SOURCES = ["attn_bf16.hip", "attn_f32.hip", "cache_ops.hip"]
HOST_SOURCES = ["ll_host.cpp"]
LIB = os.path.join(PKG, "libll.so")
FAKE_LIB = os.path.join(PKG, "libll_fake.so")
SAN_LIB = os.path.join(PKG, "libll_fake_san.so")
C_CONSUMER_SRC = os.path.join(ROOT, "tests", "c_abi_stream.c")
C_CONSUMER = os.path.join(ROOT, "tests", "c_abi_stream")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# packed-fp32 VALU ops are disabled for every HIP object (hipcc emits them on its own from
# scalar or float2 code otherwise)
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
# per-source extra flags: the attention kernels never see NaN (masking uses -inf), so IEEE
# NaN quieting of every fmaxf operand is dropped
EXTRA_FLAGS = {"attn_bf16.hip": ["-fno-honor-nans"]}
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]
# the recording host build again, instrumented with AddressSanitizer and UndefinedBehavior-
# Sanitizer (host code only; tests/test_host_sanitizers.py runs the host tests against it)
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout)
        raise RuntimeError(f"build step failed: {cmd[0]} ({r.returncode})")
    return r.stdout


def build(verbose: bool = False) -> None:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        out = _run([HIPCC, *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
                    "-o", obj])
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    shutil.move(tmp, LIB)
    # CPU-only library with the recording launch backend
    tmp = FAKE_LIB + ".tmp"
    _run(["g++", *HOST_FLAGS, "-shared", os.path.join(CSRC, "ll_host.cpp"),
          os.path.join(CSRC, "fake_launch.cpp"), "-o", tmp])
    shutil.move(tmp, FAKE_LIB)
    tmp = SAN_LIB + ".tmp"
    host_sources = [os.path.join(CSRC, "ll_host.cpp"), os.path.join(CSRC, "fake_launch.cpp")]
    _run(["g++", *HOST_FLAGS, *SAN_FLAGS, "-shared", *host_sources, "-o", tmp])
    shutil.move(tmp, SAN_LIB)
    # a plain-C program against include/ll.h and libll.so (host code only: gcc, HIP runtime API)
    tmp = C_CONSUMER + ".tmp"
    _run(["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
          "-I", os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__", C_CONSUMER_SRC,
          "-L", PKG, "-lll", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath,$ORIGIN/../windowed_attention_kv_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
          "-o", tmp])
    shutil.move(tmp, C_CONSUMER)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print("built", LIB, FAKE_LIB)

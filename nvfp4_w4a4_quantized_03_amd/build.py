"""Builds the gfx950 shared library libnvfp4_w4a4.so in the package folder.

hipcc compiles every HIP translation unit for gfx950 only, then links them
with the host-only C-ABI front end.  Flags:
  -ffp-contract=off                  no implicit fused multiply-adds
  -fno-gpu-flush-denormals-to-zero   keep binary32 subnormals (exactness)
  -target-feature -packed-fp32-ops   no packed fp32 VALU instructions
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libnvfp4_w4a4.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
          "-I" + os.path.join(ROOT, "include")]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH,
          "-fno-gpu-flush-denormals-to-zero",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = ["quantize.hip", "harmonize.hip", "gemm.hip", "gemm_stream.hip",
           "dequantize.hip", "fp8kv.hip", "api.cpp"]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DIR, src + ".o")
    flags = COMMON + (DEVICE if src.endswith(".hip") else
                      ["-D__HIP_PLATFORM_AMD__"])
    cmd = [HIPCC] + flags + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd),
                                                      r.stdout, r.stderr))
    return obj


def build(verbose=False):
    """Compile and link the library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + \
        ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout,
                                                   r.stderr))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

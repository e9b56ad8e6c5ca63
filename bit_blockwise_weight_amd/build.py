"""Build libqk.so (the HIP/gfx950 library behind include/qk.h) in-tree.

    python -m bit_blockwise_weight_amd.build        # or build() from Python

Every source is compiled with hipcc for gfx950 only:
  -ffp-contract=off                   no implicit fused multiply-add: the
                                      bit-exact steps round every product and
                                      sum on their own (explicit fmaf stays fused)
  -fno-gpu-flush-denormals-to-zero    fp32 subnormals are kept (a subnormal t
                                      can decide a code)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                      no packed fp32 VALU instructions
The library lands next to this file (bit_blockwise_weight_amd/libqk.so), and
with it libqk_probe.so: the HBM read-ceiling probe that bench.py times (not part
of the C ABI).
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqk.so")
PROBE_LIB = os.path.join(PKG, "libqk_probe.so")
PROBE_SOURCE = "hbm_probe.hip"

SOURCES = ["api.cpp", "codebook.cpp", "quantize.hip", "double_quant.hip", "dequantize.hip", "gemv.hip", "gemm.hip",
           "merge.hip", "backward.hip", "quantize8.hip", "int8mm.hip"]

COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm is required to build libqk)")
    return p


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + COMMON_FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + [
        "-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libqk.so failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    probe_obj = _compile(PROBE_SOURCE)
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, probe_obj,
           "-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libqk_probe.so failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

"""Build libqgemv.so (HIP, gfx950) in-tree: block_quantized_gemv_w4a8_amd/_lib/.

    python -m block_quantized_gemv_w4a8_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Flags that matter:
  * no fast-math: the activation quantiser needs a correctly rounded fp32
    division and roundf's half-away-from-zero rounding;
  * -fhip-fp32-correctly-rounded-divide-sqrt (the default, stated explicitly);
  * the packed-fp32 target feature is switched off, so the compiler emits no
    v_pk_{add,mul,fma}_f32 (the host pass warns that it does not know the
    feature; that warning is harmless).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIB_DIR, "libqgemv.so")

SOURCES = ["qgemv_api.cpp", "k_quantize.hip", "k_gemv.hip", "k_small_m.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # MFMA results straight into VGPRs: the small-M epilogue reads every
    # result with vector instructions, and AGPR results need a copy each
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def build(force: bool = True, verbose: bool = False) -> str:
    if not force and os.path.exists(LIB):
        return LIB
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    srcs = []
    for s in SOURCES:
        p = os.path.join(CSRC, s)
        # .cpp files include the HIP runtime: compile them as HIP as well
        srcs += (["-x", "hip", p, "-x", "none"] if s.endswith(".cpp") else [p])
    cmd = [HIPCC, *FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libqgemv.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

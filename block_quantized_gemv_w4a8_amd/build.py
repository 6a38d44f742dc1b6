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

SOURCES = ["qgemv_api.cpp", "k_quantize.hip", "k_gemv.hip", "k_gemv_q4_0.hip", "k_gemv_q4_k.hip",
           "k_gemv_q6_k.hip", "k_gemv_q6_k_r8.hip", "k_gemv_q8_0.hip", "k_small_m.hip",
           "k_small_m2.hip", "k_small_m_rows.hip", "k_small_m3.hip",
           "k_measure.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # MFMA results straight into VGPRs: the small-M epilogue reads every
    # result with vector instructions, and AGPR results need a copy each
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, obj: str, verbose: bool) -> None:
    # .cpp files include the HIP runtime: compile them as HIP as well
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, "-c", *lang, src, "-o", obj]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the library."""
    if not force and os.path.exists(LIB):
        return LIB
    from concurrent.futures import ThreadPoolExecutor
    obj_dir = os.path.join(LIB_DIR, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    tag = "%d" % os.getpid()
    objs = [os.path.join(obj_dir, os.path.splitext(s)[0] + "." + tag + ".o") for s in SOURCES]
    try:
        with ThreadPoolExecutor(len(SOURCES)) as pool:
            futs = [pool.submit(_compile, os.path.join(CSRC, s), o, verbose)
                    for s, o in zip(SOURCES, objs)]
            for f in futs:
                f.result()
        tmp = LIB + ".tmp" + tag
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed linking libqgemv.so")
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

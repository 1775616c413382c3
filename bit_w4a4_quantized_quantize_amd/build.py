"""Builds libsvdq.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each source compiles to an object under _build/ in parallel, then one link.
Usage: python -m bit_w4a4_quantized_quantize_amd.build [-v]
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libsvdq.so")

SOURCES = ["api.hip", "quant_act.hip", "quant_lora.hip", "gemm_w4a4.hip", "gemm_lds.hip", "gemm_bf16.hip",
           "repack.hip", "prep.hip", "gemm_mx.hip", "calib.hip", "gemm_bf16_blaslt.hip"]
HEADERS = ["common.h", "kernels.h"]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


COMMON_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-gpu-flush-denormals-to-zero",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        print("\n".join(noise), flush=True)
    return obj


def build(verbose=False):
    """Compile every HIP source for gfx950 and link libsvdq.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-L/opt/rocm/lib", "-lhipblaslt",
           "-Wl,-rpath,/opt/rocm/lib", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH, flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)

"""Build libqgemm.so (the HIP kernels and the C-ABI entry points) for gfx950.

Each source compiles with hipcc in parallel; the objects link into one
shared library next to this file.  Every HIP source is built with packed
fp32 instructions disabled (-target-feature -packed-fp32-ops).
"""
import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [
    "int8_tiled_256x256.hip",
    "int8_tiled_256x128.hip",
    "int8_tiled_128x128.hip",
    "int8_dma_256x256.hip",
    "int8_dma_256x128s3.hip",
    "int8_dma_128x128.hip",
    "int8_dma_128x128s3.hip",
    "int8_dma_256x256w8.hip",
    "int8_dma_256x128w8.hip",
    "int8_dma_128x128k128.hip",
    "int8_dma_256x128w8k128.hip",
    "int8_dma_256x256w8k128.hip",
    "int8_dma_64x128k128.hip",
    "a8w8_skinny.hip",
    "a8w8_slab.hip",
    "w8a32.hip",
    "w8a32_split.hip",
    "w8a32_skinny.hip",
    "dynamic_quantize.hip",
    "conv_integer.hip",
    "conv_implicit.hip",
    "calibrate.hip",
    "api.cpp",
]

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fhip-fp32-correctly-rounded-divide-sqrt",
         "-Wall", "-Wno-unused-function"]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs)
    return obj


def build_library(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))

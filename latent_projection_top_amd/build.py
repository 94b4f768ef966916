"""Build libroute.so (the route's C-ABI library) for gfx950 with hipcc, in-tree.

Every HIP source is compiled with packed FP32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass prints a
harmless warning that it does not know that feature.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libroute.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["route_api.cpp", "topk16.hip", "topk16_sharded.hip", "decode_route.hip", "prefill_gemm.hip"]
HEADERS = ["route_device.h", "route_launch.h"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]

# Per-source extra flags. The prefill GEMM keeps its MFMA accumulators in
# VGPRs (the VGPR form of v_mfma): measured on gfx950, MFMAs accumulating in
# AGPRs issued at about half the rate when a SIMD held a single wave. Its
# machine scheduler is the iterative ILP one: under the default scheduler
# the GEMMs sit at the 256-VGPR limit (the [K][N] latent GEMM spilled), with
# it they compile without spills (222-254 VGPRs), so every GEMM can spread
# its stage loads over its MFMAs, and the latent GEMMs ran 4-10 % faster
# (same bits).
EXTRA_FLAGS = {"prefill_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form",
                                    "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON_FLAGS + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


EXAMPLE_SRC = os.path.join(ROOT, "tests", "c_abi", "route_example.c")
EXAMPLE_EXE = os.path.join(BUILD_DIR, "route_example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_example(verbose: bool = False) -> str:
    """The C example (tests/c_abi/route_example.c): plain C99 over the HIP
    runtime API and libroute.so, found next to the binary's directory."""
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), EXAMPLE_SRC,
           "-L", HERE, "-lroute", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/..", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", EXAMPLE_EXE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C example failed:\n{r.stderr}")
    if verbose:
        print(f"built {EXAMPLE_EXE}", file=sys.stderr)
    return EXAMPLE_EXE


def build(verbose: bool = False) -> str:
    """Compile every source and link libroute.so next to this file, then the
    C example that links against it."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    build_example(verbose)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)

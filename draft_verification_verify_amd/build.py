"""Build libspecverify.so in-tree with hipcc for gfx950.

Every translation unit is compiled with packed-FP32 instructions disabled and
without floating-point contraction (so the same expression compiles to the same
arithmetic everywhere it is used).  The streaming-statistics kernels are built
with -fno-honor-nans (NaN logits are outside the library's contract), which
lets max() lower to bare v_max3_f32.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libspecverify.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

SOURCES = {
    "sv_stats.hip": ["-fno-honor-nans"],
    "sv_decide.hip": [],
    "sv_sample.hip": [],
    "sv_trunc.hip": [],
    "sv_api.hip": [],
}


def _compile(src: str, extra: list) -> str:
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


CEILING_SRC = os.path.join(CSRC, "sv_ceiling.hip")
CEILING_LIB = os.path.join(HERE, "libsvceiling.so")


def build_ceiling(verbose: bool = False) -> str:
    """libsvceiling.so: the plain streaming-read kernel bench.py measures the
    device's achievable read rate with (a measurement tool, not part of the
    verification library)."""
    tmp = CEILING_LIB + ".tmp"
    cmd = [HIPCC, *COMMON, "-shared", CEILING_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for sv_ceiling.hip:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CEILING_LIB)
    if verbose:
        print("built", CEILING_LIB)
    return CEILING_LIB


CLIENT_SRC = os.path.join(ROOT, "tests", "c_client", "sv_client.c")
CLIENT_BIN = os.path.join(ROOT, "tests", "c_client", "sv_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_client(verbose: bool = False) -> str:
    """The plain C client of the boundary (tests/c_client): gcc, C99, linked
    against libspecverify.so and the HIP runtime, no Python or torch."""
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
           f"-I{ROCM}/include", CLIENT_SRC, "-o", CLIENT_BIN, f"-L{HERE}", "-lspecverify",
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,$ORIGIN/../../draft_verification_verify_amd",
           f"-Wl,-rpath,{ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"client build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print("built", CLIENT_BIN)
    return CLIENT_BIN


if __name__ == "__main__":
    build(verbose=True)
    build_ceiling(verbose=True)
    build_client(verbose=True)

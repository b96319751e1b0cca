"""Builds libaq.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m weight_only_bit_group_amd.build        # or build() from Python

Every call recompiles all sources.  Objects go to ``_build/`` at the repository
root; the shared library is written next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libaq.so")
# the ceiling microbenchmarks the benchmark runs beside the path (not part of the C ABI)
PROBE_SOURCE = os.path.join(CSRC, "probe", "ceiling.hip")
PROBE_PATH = os.path.join(HERE, "libaq_probe.so")

HIP_SOURCES = ("quant_pack.hip", "w4a16_gemv.hip", "decode_mfma.hip", "mfma_gemm.hip", "act_absmean.hip",
               "awq_search.hip", "fp4_gemv.hip", "fp4_quant.hip", "w8a16_gemv.hip")
CPP_SOURCES = ("aq_api.cpp",)

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # Bit-exact quantization: IEEE division, no contraction into FMAs, no fast-math,
    # fp32 denormals preserved.
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    # Keep the compiler from forming packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I" + os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libaq)")


# Per-file extra flags: the GEMMs keep MFMA accumulators in VGPRs (the fp32
# group rescale operates on them with plain VALU FMAs).
FILE_FLAGS = {"mfma_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{proc.stdout}\n{proc.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source for gfx950 and link libaq.so; returns the library path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    sources = list(HIP_SOURCES) + list(CPP_SOURCES)
    jobs = min(len(sources) + 1, max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        probe_obj = pool.submit(_compile, PROBE_SOURCE)
        objs = list(pool.map(_compile, sources))
        probe_obj = probe_obj.result()
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{proc.stdout}\n{proc.stderr}")
    os.replace(tmp, LIB_PATH)
    tmp = PROBE_PATH + ".tmp"
    proc = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", probe_obj, "-o", tmp],
                          capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"probe link failed:\n{proc.stdout}\n{proc.stderr}")
    os.replace(tmp, PROBE_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()
    sys.exit(0)

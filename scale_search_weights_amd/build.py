"""Build libnvfp4.so (the HIP kernels and the C ABI) for gfx950, in-tree.

``python -m scale_search_weights_amd.build`` or ``build()`` from Python. Every call
recompiles: objects go to ``_build/`` and the library to the package directory.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libnvfp4.so")
PROBE_OUT = os.path.join(PKG, "libnvfp4_probe.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["nvfp4_api.hip", "nvfp4_quant.hip", "nvfp4_search.hip", "nvfp4_hessian.hip",
           "nvfp4_calib.hip", "nvfp4_ste.hip", "nvfp4_gram.hip", "nvfp4_gptq.hip", "nvfp4_debug.hip",
           "nvfp4_noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # exact rounding decisions: no contraction, keep fp32 denormals
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 ops in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs (no accumulator-register copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    os.makedirs(os.path.dirname(obj), exist_ok=True)
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    # peak-rate probes used by the benchmark only (a separate library, not the C ABI)
    pobj = _compile(os.path.join("probe", "nvfp4_probe.hip"))
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", pobj, "-o", PROBE_OUT + ".tmp"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(PROBE_OUT + ".tmp", PROBE_OUT)
    if verbose:
        print("built", PROBE_OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

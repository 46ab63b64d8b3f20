"""Builds libkvq.so for gfx950 in-tree with hipcc (no JIT, no torch extension).

    python -m bit_kv_cache_block_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "kvq")
LIB = os.path.join(PKG, "libkvq.so")
# memory-system ceiling probes for the benchmark (not part of the C ABI)
PROBE_LIB = os.path.join(PKG, "libkvq_probe.so")
PROBE_SOURCES = ["probe.hip"]

SOURCES = ["api.cpp", "append.hip", "decode_int4.hip", "decode_int4_sk.hip", "decode_mxfp4.hip", "decode_bf16.hip", "decode_windowed.hip", "reduce.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # quantizer steps are rounded one operation at a time (no contraction)
    "-ffp-contract=off",
    # no packed-fp32 instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: their results feed VALU code directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

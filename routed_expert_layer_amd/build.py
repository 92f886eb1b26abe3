"""Build libmb.so (the gfx950 HIP kernels and the C ABI of include/mb.h) in-tree.

Run: python -m routed_expert_layer_amd.build
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmb.so")
# The HBM read probe bench.py --read-probe times (not part of libmb.so).
PROBE_SRC = "read_probe.hip"
PROBE_LIB = os.path.join(PKG, "libmb_readprobe.so")
SOURCES = ["api.hip", "block.hip", "block_w4a4.hip", "block_qkv.hip", "block_w4a4_qkv.hip", "block_many.hip", "route.hip", "gemm_bf16.hip", "experts.hip", "boundary.hip", "pack.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # Packed fp32 VALU ops stay off: the compiler emits plain fp32 arithmetic.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division and square root (the route weights are fp32 quotients).
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-I", CSRC,
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    # -z defs: an unresolved symbol fails the link rather than the first call.
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libmb.so (and the read
    probe's library); returns libmb.so's path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + [PROBE_SRC]))
    _link(objs[-1:], PROBE_LIB)
    objs = objs[:-1]
    _link(objs, LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

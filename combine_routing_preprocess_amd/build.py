"""Build libmoe_route.so (HIP for gfx950) in-tree.

Usage: python -m combine_routing_preprocess_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_route.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "ring.cpp", "route.hip", "permute.hip", "combine.hip", "backward.hip", "gemm_bf16.hip", "gemm_fp8.hip", "noalloc.hip", "decode.hip", "decode_fused.hip"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
          "-Wno-inline-asm"]


def _compile(src: str, out_dir: str = OUT_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = True, lib_path: str = LIB, extra=()) -> str:
    """Compile every source and link the shared library.  ``extra`` adds
    compiler flags (e.g. -D overrides of compile-time tile parameters) and
    ``lib_path`` redirects the output for such variant builds."""
    out_dir = OUT_DIR if lib_path == LIB else os.path.join(os.path.dirname(lib_path), "_build")
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir, extra), SOURCES))
    LIBP = lib_path
    tmp = LIBP + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs + ["-Wl,--no-undefined"]
    subprocess.check_call(cmd)
    os.replace(tmp, LIBP)
    if verbose:
        print(f"built {LIBP}")
    return LIBP


if __name__ == "__main__":
    build()

"""Build the HIP library in-tree: strided_fp32_gemm_amd/libsgemm_strided.so.

    python -m strided_fp32_gemm_amd.build            # compile for gfx950
    python -m strided_fp32_gemm_amd.build --asm DIR  # also keep device assembly

hipcc cross-compiles gfx950 code objects on a host without a GPU.  Every HIP
source is built with the packed-fp32 target feature turned off, so the
compiler never emits packed fp32 add/mul/fma instructions.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libsgemm_strided.so")
BUILD_DIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
SOURCES = ["plan.cpp", "attention.cpp", "splitk.cpp", "abi.cpp", "kernels.hip", "attn_kernel.hip",
           "strip_kernel.hip", "splitk_kernel.hip", "attn_splitkv_kernel.hip", "scratch.hip"] + [f"mfma_t{t}.hip" for t in range(13)] + \
    [f"wave_w{t}.hip" for t in range(8)] + [f"persist_p{t}.hip" for t in range(3)]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, asm_dir: str | None) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    if asm_dir and src.endswith(".hip"):
        os.makedirs(asm_dir, exist_ok=True)
        asm = os.path.join(asm_dir, os.path.splitext(src)[0] + f"-{ARCH}.s")
        subprocess.run([_hipcc(), "-x", "hip", *common_flags(), "--cuda-device-only", "-S",
                        os.path.join(CSRC, src), "-o", asm], check=True, capture_output=True)
    return obj


def build(asm_dir: str | None = None, verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm_dir), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="directory for device assembly listings")
    args = ap.parse_args()
    build(args.asm, verbose=True)


if __name__ == "__main__":
    main()

"""Build libvqmm.so in-tree with hipcc for gfx950.

    python -m compressed_index_matmul_amd.build [--jobs N] [--verbose]

Every HIP translation unit is compiled for gfx950 only, with packed-FP32
instruction selection disabled, then linked into one shared library next to
this file.  Rebuilds from scratch each time (a few tens of seconds).
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvqmm.so")
ARCH = "gfx950"

SOURCES = ["vqmm_api.cpp", "k_dequant.hip", "k_rht.hip", "k_gemv.hip", "k_gemv_ladder.hip", "k_gemm.hip",
           "k_gemm_ladder.hip", "k_sparse.hip",
           "k_gemv_sparse.hip", "k_gemv_l2.hip", "k_gemv_cbs.hip", "k_lowrank.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libvqmm")
    return p


def _compile(src: str, obj: str, verbose: bool) -> None:
    cmd = [hipcc(), *COMMON_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(jobs: int = 0, verbose: bool = False) -> str:
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with tempfile.TemporaryDirectory(prefix="vqmm_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
            futs = [ex.submit(_compile, s, o, verbose) for s, o in zip(SOURCES, objs)]
            for f in futs:
                f.result()
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp_lib, LIB)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()

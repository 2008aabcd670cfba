"""Build libvqmm.so in-tree with hipcc for gfx950.

    python -m compressed_index_matmul_amd.build [--jobs N] [--verbose]
    python -m compressed_index_matmul_amd.build --hostsan   (CPU-test build)

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


# ---------------------------------------------------------------------------
# Host-sanitized build for the CPU tests: the same sources, host code only,
# with AddressSanitizer and UndefinedBehaviorSanitizer on the host side.  No
# device code is compiled: every translation unit embeds an empty GPU binary,
# so the library loads and validates arguments but can launch nothing.  It
# is loaded by a Python started with the clang ASan runtime preloaded
# (hostsan_env) and VQMM_LIBRARY naming it.
# ---------------------------------------------------------------------------
HOSTSAN_DIR = os.path.join(HERE, "_hostsan")
HOSTSAN_LIB = os.path.join(HOSTSAN_DIR, "libvqmm_hostsan.so")
HOSTSAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The clang ASan runtime that matches hipcc's host compiler."""
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm", "lib", "clang")
    if not os.path.isdir(root):
        root = "/opt/rocm/llvm/lib/clang"
    for ver in sorted(os.listdir(root), reverse=True):
        p = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise RuntimeError(f"no libclang_rt.asan-x86_64.so under {root}")


def hostsan_env(base=None) -> dict:
    """Environment of a process that loads the host-sanitized library."""
    env = dict(os.environ if base is None else base)
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["VQMM_LIBRARY"] = HOSTSAN_LIB
    return env


def _compile_hostsan(src: str, obj: str, empty_bin: str) -> None:
    cmd = [hipcc(), "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "--offload-host-only",
           "-Xclang", "-fcuda-include-gpubinary", "-Xclang", empty_bin, *HOSTSAN_FLAGS,
           "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"host-sanitized compile failed on {src}:\n{err}")


def build_hostsan(jobs: int = 0) -> str:
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    os.makedirs(HOSTSAN_DIR, exist_ok=True)
    with tempfile.TemporaryDirectory(prefix="vqmm_hostsan_") as tmp:
        empty = os.path.join(tmp, "empty.bin")
        open(empty, "wb").close()
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
            for f in [ex.submit(_compile_hostsan, s, o, empty) for s, o in zip(SOURCES, objs)]:
                f.result()
        tmp_lib = HOSTSAN_LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "--offload-host-only", "-shared", "-fPIC", *HOSTSAN_FLAGS,
               "-Xarch_host", "-shared-libasan", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"host-sanitized link failed:\n{r.stderr}")
        os.replace(tmp_lib, HOSTSAN_LIB)
    return HOSTSAN_LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--hostsan", action="store_true", help="build the host-sanitized library for the CPU tests")
    args = ap.parse_args()
    print(build_hostsan(args.jobs) if args.hostsan else build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()

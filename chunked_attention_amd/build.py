"""Build the HIP library libkvc.so (gfx950) in-tree, plus the CPU-only test
build of the host logic.

    python -m chunked_attention_amd.build          # device library
    python -m chunked_attention_amd.build --host   # CPU test library too

The device library always compiles from scratch.  Every HIP translation unit
is built with packed-FP32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops).
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvc.so")
HOST_LIB = os.path.join(BUILD, "libkvc_hostcheck.so")
HOST_LIB_SAN = os.path.join(BUILD, "libkvc_hostcheck_san.so")
# AddressSanitizer + UndefinedBehaviorSanitizer for the CPU test build of the
# host logic (g++ only: no device code is built with them).  A process that
# loads it must preload the ASan runtime (asan_runtime()).
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]

HIP_SOURCES = ["cache_write.hip", "attn_fwd.hip", "attn_fwd_fp8.hip", "edit_mask.hip",
               "noalloc.hip"]
CPP_SOURCES = ["ring.cpp", "plan.cpp"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
# Per-source extra flags: LLVM scheduling strategies measured on MI355X (same
# results bit for bit).  bf16 kernel: max-memory-clause, 1.9% faster than the
# default schedule.  fp8 kernel: max-ilp, 0.9% faster at 40 heads and 6% at 8
# (it halves the spills of the piece prologue and merge).
SOURCE_FLAGS = {
    "attn_fwd.hip": ["-mllvm", "--amdgpu-sched-strategy=max-memory-clause"],
    "attn_fwd_fp8.hip": ["-mllvm", "--amdgpu-sched-strategy=max-ilp"],
}


def _run(cmd: list[str], verbose: bool, cwd: str | None = None) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=cwd)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    if verbose and (r.stdout.strip() or r.stderr.strip()):
        # hipcc's host pass warns about the target feature it does not know
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l and l.strip())
        if msg:
            print(msg)


def hip_sources() -> list[str]:
    return [s for s in HIP_SOURCES if os.path.exists(os.path.join(CSRC, s))]


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    """Compile libkvc.so for gfx950 into the package directory."""
    objdir = os.path.join(BUILD, "obj")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for src in hip_sources():
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), f"-I{INCLUDE}", "-c",
               os.path.join(CSRC, src), "-o", obj]
        cwd = None
        if save_temps:
            cwd = os.path.abspath(save_temps)
            os.makedirs(cwd, exist_ok=True)
            cmd.insert(1, "-save-temps")
        jobs.append((cmd, obj, cwd))
    for src in CPP_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        jobs.append((["g++", *CXX_FLAGS, f"-I{INCLUDE}", "-c", os.path.join(CSRC, src),
                      "-o", obj], obj, None))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda j: _run(j[0], verbose, j[2]), jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
          *[o for _, o, _ in jobs]], verbose)
    os.replace(tmp, LIB)
    return LIB


def build_host(verbose: bool = False, sanitize: bool = False) -> str:
    """CPU-only library of the host logic (ring, ABI, plan) linked against the
    recording test launcher in tests/; with sanitize, built with ASan and
    UBSan into HOST_LIB_SAN."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in CPP_SOURCES]
    srcs.append(os.path.join(ROOT, "tests", "fake_launch.cpp"))
    out = HOST_LIB_SAN if sanitize else HOST_LIB
    tmp = out + ".tmp"
    flags = CXX_FLAGS + (SAN_FLAGS if sanitize else [])
    _run(["g++", *flags, f"-I{INCLUDE}", f"-I{CSRC}", "-shared", "-o", tmp, *srcs], verbose)
    os.replace(tmp, out)
    return out


def asan_runtime() -> str:
    """Path of the ASan runtime g++ links against (for LD_PRELOAD)."""
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    return os.path.realpath(r.stdout.strip())


def host_lib_stale(path: str = HOST_LIB) -> bool:
    if not os.path.exists(path):
        return True
    t = os.path.getmtime(path)
    deps = [os.path.join(CSRC, s) for s in os.listdir(CSRC)]
    deps += [os.path.join(INCLUDE, "kvc.h"), os.path.join(ROOT, "tests", "fake_launch.cpp"),
             os.path.join(ROOT, "tests", "e4m3_rule.hpp"), os.path.abspath(__file__)]
    return any(os.path.getmtime(p) > t for p in deps if os.path.exists(p))


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--host", action="store_true", help="also build the CPU test library")
    ap.add_argument("--save-temps", default=None, help="directory for ISA dumps")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.verbose, args.save_temps))
    if args.host:
        print(build_host(args.verbose))


if __name__ == "__main__":
    main()

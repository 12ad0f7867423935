"""Build libmoe.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

Usage: python -m quantized_moe_expert_02_amd.build  [--jobs N]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe.so")
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ["moe_api.hip", "route.hip", "router_gemm.hip", "permute.hip", "expert_gemv.hip",
           "expert_gemm.hip", "expert_gemm_d.hip", "expert_gemm_q.hip", "quantize.hip", "decode.hip", "combine.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in device code.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmoe.so")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build failed: " + " ".join(cmd))
    return r


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    missing = [s for s in SOURCES if not os.path.exists(os.path.join(CSRC, s))]
    if missing:
        raise RuntimeError("missing sources: " + ", ".join(missing))
    srcs = SOURCES

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        return obj

    n = jobs or min(len(srcs), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(max_workers=n) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(driver: str, out_dir: str, jobs: int | None = None) -> str:
    """Every library source plus a host test driver, with AddressSanitizer and
    UndefinedBehaviorSanitizer on the host code only (the device code is
    built as usual; the driver exercises validation, workspace planning and
    argument checks, and never launches).  Returns the executable's path."""
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", *san]

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.basename(src).rsplit(".", 1)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([cc, *flags, *lang, "-c", src, "-o", obj])
        return obj

    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [driver]
    n = jobs or min(len(srcs), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(max_workers=n) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = os.path.join(out_dir, "host_checks")
    _run([cc, f"--offload-arch={ARCH}", *san, "-o", exe, *objs])
    return exe


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))

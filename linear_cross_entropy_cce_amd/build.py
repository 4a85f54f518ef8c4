"""Builds libcce.so (gfx950 HIP kernels + the C ABI) in-tree with hipcc.

    python -m linear_cross_entropy_cce_amd.build [--debug] [--host-check]

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection turned off (-Xclang -target-feature -Xclang -packed-fp32-ops).

--host-check also builds _build/host_check/abi_check: the C ABI's host code
(api.cpp) and the argument-check driver tests/abi_check.cpp compiled with
AddressSanitizer and UndefinedBehaviorSanitizer on the host side only
(device code is built as usual), linked with the kernels' objects.
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
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libcce.so")

HIP_SOURCES = ["fwd.hip", "bwd.hip", "vsort.hip"]
CPP_SOURCES = ["api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return err


def build(debug: bool = False, verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    common = ["-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
              "-Wall", "-Wno-unused-function"]
    common += ["-O1", "-g"] if debug else ["-O3"]
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append([cc, *common, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append([cc, *common, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for msg in ex.map(_compile, jobs):
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    subprocess.run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def build_host_check(verbose: bool = False) -> str:
    """The sanitized host-check program (see the module docstring); needs the
    kernels' objects of a normal build (made here if absent)."""
    cc = hipcc()
    objs = [os.path.join(BUILD_DIR, src + ".o") for src in HIP_SOURCES]
    if not all(os.path.exists(o) for o in objs):
        build(verbose=verbose)
    out_dir = os.path.join(BUILD_DIR, "host_check")
    os.makedirs(out_dir, exist_ok=True)
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]  # host side only
    common = ["-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC, "-Wall",
              "-Wno-unused-function", "-O1", "-g", "-fno-omit-frame-pointer", *host_san]
    api_o = os.path.join(out_dir, "api.o")
    drv_o = os.path.join(out_dir, "abi_check.o")
    _compile([cc, *common, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o])
    _compile([cc, *common, "-c", os.path.join(ROOT, "tests", "abi_check.cpp"), "-o", drv_o])
    exe = os.path.join(out_dir, "abi_check")
    subprocess.run([cc, f"--offload-arch={ARCH}", *host_san, drv_o, api_o, *objs, "-o", exe], check=True)
    return exe


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--host-check", action="store_true")
    a = ap.parse_args()
    print(build(debug=a.debug, verbose=a.verbose))
    if a.host_check:
        print(build_host_check(verbose=a.verbose))

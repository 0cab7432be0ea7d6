"""Build libdflash.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m block_diffusion_drafter_forward_amd.build [--force]
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libdflash.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("DFLASH_ARCH", "gfx950")

HIP_SOURCES = ["gemm.hip", "attention.hip", "head.hip", "elementwise.hip", "ddtree.hip", "spec_verify.hip", "tree_attn.hip",
               "scratch.hip"]
CPP_SOURCES = ["dflash_api.cpp"]

COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Packed fp32 VALU ops are kept out of the generated code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def _needs_rebuild(obj, deps):
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def build(force: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    headers = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    headers.append(os.path.join(INCLUDE, "dflash.h"))
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        s = os.path.join(CSRC, src)
        o = os.path.join(BUILD_DIR, src + ".o")
        objs.append(o)
        if force or _needs_rebuild(o, [s] + headers):
            jobs.append([hipcc, "-x", "hip", "-c", s, "-o", o] + COMMON + DEVICE)
    for src in CPP_SOURCES:
        s = os.path.join(CSRC, src)
        o = os.path.join(BUILD_DIR, src + ".o")
        objs.append(o)
        if force or _needs_rebuild(o, [s] + headers):
            # (the same target as the kernels: headers they share hold gfx950-only device code)
            jobs.append([hipcc, "-c", s, "-o", o, "-D__HIP_PLATFORM_AMD__"] + COMMON + DEVICE)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, max(1, len(jobs)))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    if force or jobs or not os.path.exists(OUT):
        tmp = OUT + ".tmp"
        _run([hipcc, "-shared", "-o", tmp] + objs + [f"--offload-arch={ARCH}", "-fPIC"])
        os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(force="--force" in sys.argv, verbose=True))

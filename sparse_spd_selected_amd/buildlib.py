"""Compile libselinv.so (HIP, gfx950 only) in place.

Every HIP translation unit is built with hipcc for gfx950 with packed-fp32
instructions disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libselinv.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = [
    "abi.cpp",
    "tree_plan.cpp",
    "generic.hip",
    "chain_b16.hip",
    "star_b32.hip",
    "chain_b32.hip", "chain_b32_seg.hip",
    "tree_b8.hip",
    "chain_small.hip", "chain_noalloc.hip",
    "vjp_generic.hip", "vjp_chain_b16.hip", "vjp_star_b32.hip",
    "vjp_tree_b8.hip", "vjp_chain_seg.hip",
    "shared_factor.hip", "chain_solve_b16.hip", "star_solve_b32.hip",
    "nonsym.hip", "bidiag_b16.hip", "nonsym_b8.hip", "junction_plan.cpp", "junction.hip",
    "junction_solve.hip",
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]
# device code: gfx950 only; packed FP32 vector instructions disabled
HIP_FLAGS = ["-x", "hip", "--offload-arch=" + ARCH,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]


def _compile(src: str, build_dir: str = BUILD_DIR, host_flags=()) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON_FLAGS + list(host_flags)
    if src.endswith(".hip"):
        cmd += HIP_FLAGS
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = False, out: str = LIB, build_dir: str = BUILD_DIR,
          host_flags=()) -> str:
    """Compile every source and link `out`.  `host_flags` go to the host side
    of every compile and to the link (the tests use it for a host-sanitizer
    build of the library in its own build_dir)."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, host_flags), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + list(host_flags) + \
        ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

"""Builds libtree_attn.so in-tree with hipcc for gfx950.

Usage: ``python -m prefix_shared_tree_attn_amd.build`` (or ``build()``).
Objects go to ``_build/`` next to this file; the shared library is written
next to this file so that the binding loads it from the package directory.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtree_attn.so")
ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

SOURCES = ["api.cpp", "planner.cpp", "prefix_tree.cpp", "fwd.hip", "bwd.hip", "positions.hip",
           "prefix_ops.hip", "linear.hip", "scratch.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: the packed fp32 instructions are disabled (the compiler would
# otherwise form them from ordinary float code).  The kernels use no atomics.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
DEVICE = [f"--offload-arch={ARCH}", *DEVICE_FLAGS]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
    else:
        cmd += ["-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every source and links ``libtree_attn.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host sanitizer build: the host sources (planner, prefix-tree builder, C
# ABI) compiled by the host compiler with AddressSanitizer and
# UndefinedBehaviorSanitizer, linked with the regular device objects.  Only
# host code is instrumented; no GPU code is built with a sanitizer.
HOST_SOURCES = ["api.cpp", "planner.cpp", "prefix_tree.cpp"]
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(BUILD, "libtree_attn_hostsan.so")
DEVICE_OBJECTS = [s + ".o" for s in SOURCES if s.endswith(".hip")]


def build_host_sanitized(verbose: bool = False) -> str:
    """Builds ``_build/libtree_attn_hostsan.so`` (see above) and returns its
    path.  Load it with TREE_ATTN_LIBRARY set to that path and the sanitizer
    runtime preloaded (LD_PRELOAD of the compiler's libasan)."""
    if not all(os.path.exists(os.path.join(BUILD, o)) for o in DEVICE_OBJECTS):
        build(verbose)
    out_dir = os.path.join(BUILD, "hostsan")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        cmd = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__",
               f"-I{ROCM}/include", f"-I{INCLUDE}", f"-I{CSRC}", "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"sanitizer build of {src} failed:\n{res.stderr}")
        objs.append(obj)
    cmd = ["g++", "-shared", *SAN_FLAGS, "-o", SAN_LIB, *objs,
           *[os.path.join(BUILD, o) for o in DEVICE_OBJECTS], f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{ROCM}/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitizer link failed:\n{res.stderr}")
    return SAN_LIB


if __name__ == "__main__":
    if "--host-sanitizers" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))

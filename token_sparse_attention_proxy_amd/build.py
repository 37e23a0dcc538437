"""Build libtsa.so in-tree with hipcc for gfx950.

Usage: ``python -m token_sparse_attention_proxy_amd.build`` (or ``build()``).
Every call recompiles; objects go to ``_build/`` beside this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtsa.so")
PROBE_LIB = os.path.join(PKG, "libtsa_probe.so")   # the MFMA ceiling probe (include/tsa_probe.h)

SOURCES = ["tsa_api.cpp", "score.hip", "budget.hip", "select.hip", "gather_scatter.hip",
           "attention.hip"]
PROBE_SOURCES = ["probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# the C compiler of the same LLVM (its sanitizer runtimes match hipcc's host code)
CLANG = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "llvm", "bin",
                     "clang")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


# Host code only: the GPU code of a sanitized translation unit is built as usual.
HOST_SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=undefined "
                 "-Xarch_host -fno-omit-frame-pointer").split()


def build_host_sanitized(out_dir: str) -> str:
    """Link ``libtsa_hostsan.so`` in ``out_dir``: the C-ABI translation unit
    (validation, workspace layout, launch sequencing) compiled with
    AddressSanitizer and UndefinedBehaviorSanitizer on its host code, and the
    kernel objects of the last ``build()``.  A program that loads it must be
    linked with the sanitizer runtimes (clang ``-fsanitize=address,undefined``)."""
    kernels = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES
               if s != "tsa_api.cpp"]
    missing = [o for o in kernels if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"kernel objects missing ({missing[0]}); run "
                           "`python -m token_sparse_attention_proxy_amd.build` first")
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, "tsa_api_hostsan.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SANITIZE
    cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, "tsa_api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    lib = os.path.join(out_dir, "libtsa_hostsan.so")
    _link([obj, *kernels], lib)
    return lib


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

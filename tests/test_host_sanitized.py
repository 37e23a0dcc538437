"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C-ABI translation unit (validation, workspace layout and launch sequencing)
is rebuilt with both sanitizers on its host code and driven by
``tests/abi_host_check.c``: every entry point with bad problems, null and
misaligned pointers, short or misaligned workspaces and bad ``kv_group``
values; the size queries over shapes up to the limits (L = 2^22, Hq = 4096,
B*Hq = 61440); and valid problems with the launch failure injected from the
host (``TSA_FAULT_INJECT=launch``), so that no call reaches the GPU runtime.
Runs on the CPU.
"""
from __future__ import annotations

import os
import subprocess

from token_sparse_attention_proxy_amd import build as tsa_build

HERE = os.path.dirname(os.path.abspath(__file__))


def _kernel_objects_current() -> bool:
    """The normal build's objects exist and are newer than their sources and headers."""
    heads = [os.path.join(tsa_build.CSRC, h) for h in os.listdir(tsa_build.CSRC) if h.endswith(".h")]
    heads += [os.path.join(tsa_build.INCLUDE, h) for h in os.listdir(tsa_build.INCLUDE)]
    newest_head = max(os.path.getmtime(h) for h in heads)
    for src in tsa_build.SOURCES:
        obj = os.path.join(tsa_build.BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj):
            return False
        t = os.path.getmtime(obj)
        if t < os.path.getmtime(os.path.join(tsa_build.CSRC, src)) or t < newest_head:
            return False
    return True


def test_host_code_under_sanitizers(tmp_path):
    out = str(tmp_path)
    if not _kernel_objects_current():
        tsa_build.build()
    tsa_build.build_host_sanitized(out)
    exe = os.path.join(out, "abi_host_check")
    cmd = [tsa_build.CLANG, "-O1", "-g", "-std=c11", "-Wall", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-I", tsa_build.INCLUDE,
           os.path.join(HERE, "abi_host_check.c"), "-o", exe,
           f"-L{out}", "-ltsa_hostsan", f"-Wl,-rpath,{out}", "-lpthread", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"driver build failed:\n{r.stdout}\n{r.stderr}"
    env = dict(os.environ)
    # Leak checking is off: the GPU runtime the library links keeps allocations
    # until exit.  verify_asan_link_order=0 tolerates a preloaded library ahead
    # of the runtime.
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert " 0 failures" in r.stdout, r.stdout
    n = int(r.stdout.split()[0])
    assert n > 10000, r.stdout

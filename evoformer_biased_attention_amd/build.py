"""Build libevoattn.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python -m evoformer_biased_attention_amd.build   (or build() from Python)
       python -m evoformer_biased_attention_amd.build --asan
           also libevoattn_asan.so: the same library with its host code built
           under AddressSanitizer and UndefinedBehaviorSanitizer (device code
           as in the plain build), for the host-side checks on the CPU; it
           runs with clang's ASan runtime preloaded (ASAN_RUNTIME).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libevoattn.so")
LIB_ASAN = os.path.join(HERE, "libevoattn_asan.so")
# the sanitizers apply to the host pass only (each flag right after -Xarch_host)
HOST_SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
ASAN_RUNTIME = next(iter(sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))), "")
SOURCES = ["evo_api.hip", "evo_fwd.hip", "evo_bwd.hip", "evo_bwd_tile.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU ops stay off: they are emitted by hand nowhere and the
    # compiler is told not to form them either
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _build(lib: str, objdir: str, extra, verbose: bool) -> str:
    os.makedirs(objdir, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        for src in SOURCES:
            obj = os.path.join(objdir, src.replace(".hip", ".o"))
            objs.append(obj)
            jobs.append(ex.submit(_run, [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]))
        for j in jobs:
            out = j.result()
            if verbose and out.strip():
                print(out)
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-o", tmp, *objs])
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    return _build(LIB, os.path.join(HERE, "_build"), [], verbose)


def build_asan(verbose: bool = False) -> str:
    return _build(LIB_ASAN, os.path.join(HERE, "_build_asan"), ["-g", "-fno-omit-frame-pointer", *HOST_SANITIZE],
                  verbose)


def asan_is_stale() -> bool:
    """True when libevoattn_asan.so is missing or older than a source."""
    if not os.path.exists(LIB_ASAN):
        return True
    t = os.path.getmtime(LIB_ASAN)
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    return any(os.path.getmtime(f) > t for f in srcs)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--asan" in sys.argv:
        print(build_asan(verbose="-v" in sys.argv))

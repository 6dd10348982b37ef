"""Build ``libflattn.so`` from ``csrc/*.hip`` with hipcc for gfx950.

Each translation unit compiles in its own hipcc process (in parallel); the
objects are linked into one shared library next to this file.  Run as
``python -m flashattention_attention_variants_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libflattn.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 arithmetic stays off in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _check_stubs(objs: list[str]) -> None:
    """Every kernel launch stub an object references must be defined in it
    (clang can drop a stub silently when the host pass rejects a kernel)."""
    for o in objs:
        r = subprocess.run(["nm", o], capture_output=True, text=True)
        missing = [l.split()[-1] for l in r.stdout.splitlines()
                   if l.split()[0] == "U" and "__device_stub__" in l]
        if missing:
            raise RuntimeError("%s: kernel stubs not emitted: %s" % (o, ", ".join(missing[:3])))


def build(jobs: int | None = None, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every HIP source and link the library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 8))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra or []), srcs))
    _check_stubs(objs)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])

"""Build ``libflattn.so`` from ``csrc/*.hip`` with hipcc for gfx950.

Each translation unit compiles in its own hipcc process (in parallel); the
objects are linked into one shared library next to this file.  Run as
``python -m flashattention_attention_variants_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
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
    # -save-temps=obj leaves the device assembly next to the object for the
    # register check below
    cmd = [HIPCC, *FLAGS, *extra, "-save-temps=obj", "-c", src, "-o", obj]
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


def _check_asm_loads(asm: str) -> None:
    """Inline assembly in the kernels may issue loads only into LDS
    (buffer_load ... lds, which writes no register): a load written in
    inline assembly whose destination is a register would leave that
    register's write in flight behind the compiler's back.  Fail on any
    register-destination load inside an inline-assembly region."""
    in_asm, kernel = False, ""
    with open(asm) as fh:
        for n, line in enumerate(fh, 1):
            t = line.strip()
            if re.match(r"^_Z\S+:", t):
                kernel = t
            if t.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if t.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if not in_asm or not t or t[0] in ";.":
                continue
            op = t.split()[0]
            loads = op.startswith(("ds_read", "global_load", "flat_load", "scratch_load",
                                   "buffer_load", "s_load", "s_buffer_load"))
            if loads and not (op.startswith("buffer_load") and t.rstrip().endswith(" lds")):
                raise RuntimeError("%s:%d: register-destination load in inline assembly: %s "
                                   "(in %s)" % (asm, n, t, kernel[:90]))


def build(jobs: int | None = None, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every HIP source and link the library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 8))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra or []), srcs))
    _check_stubs(objs)
    for o in objs:
        for asm in glob.glob(o[:-2] + "-hip-amdgcn-amd-amdhsa-*.s"):
            _check_asm_loads(asm)
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

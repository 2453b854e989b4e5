"""Build librha.so (gfx950) in-tree with hipcc.

Usage: ``python -m linear_attention_video_chunked_amd.build`` or
``linear_attention_video_chunked_amd.build.build()``.  Objects are compiled in
parallel under ``_build/`` and linked into ``librha.so`` next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "librha.so")
ARCH = "gfx950"

# Packed-fp32 VALU ops are disabled for all device code (the compiler would
# otherwise form v_pk_* fp32 instructions from ordinary float code).
# Private arrays are not promoted to LDS: a promoted array is addressed by the
# flat thread index, for which every workgroup first reads its dispatch packet;
# on the MI355X those reads spread the start of a launch's first 256
# workgroups over 12.5 us (0.3 us without them; measured on the split forward
# of a streaming step).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-disable-promote-alloca-to-lds"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-result"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librha)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose: bool = True, jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link librha.so; returns its path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        out = _run([cc, *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj])
        return src, out

    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        for src, out in ex.map(compile_one, zip(srcs, objs)):
            if verbose:
                print(f"[librha] compiled {os.path.relpath(src, ROOT)}", flush=True)
                warn = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip())
                if warn:
                    print(warn, flush=True)
    tmp = LIB_PATH + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"[librha] linked {os.path.relpath(LIB_PATH, ROOT)}", flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

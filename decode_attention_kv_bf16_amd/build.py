"""Build libdecode_attn.so in-tree with hipcc for gfx950.

Usage: python -m decode_attention_kv_bf16_amd.build   (or call build()).
Each HIP source is compiled to an object under _build/ in parallel, then the
objects are linked into decode_attention_kv_bf16_amd/libdecode_attn.so.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libdecode_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    # compiler-generated packed fp32 math is switched off (device code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature flag; drop that note
    lines = [ln for ln in p.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return p.returncode, "\n".join(lines)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source and link the shared library. Returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        return src, _run([cc, *COMMON_FLAGS, "-c", src, "-o", obj])

    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(compile_one, zip(srcs, objs)))
    failed = False
    for src, (rc, out) in results:
        if out.strip() and (verbose or rc != 0):
            print(f"[{os.path.basename(src)}]\n{out}", file=sys.stderr)
        failed |= rc != 0
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = LIB_PATH + ".tmp"
    rc, out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)

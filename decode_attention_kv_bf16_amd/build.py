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
# per-kernel register, spill and scratch figures that the compiler reported
# for the last build (kernel-resource-usage remarks)
RESOURCES_PATH = os.path.join(BUILD_DIR, "kernel_resources.json")

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


def parse_resource_usage(text: str) -> dict:
    """{kernel symbol: {field: int}} from the compiler's kernel-resource-usage
    remarks ("Function Name: X", then "VGPRs: n", "ScratchSize [bytes/lane]: n", ...)."""
    out, cur = {}, None
    for ln in text.splitlines():
        if "remark:" not in ln:
            continue
        body = ln.split("remark:", 1)[1].split("[-Rpass-analysis")[0].strip()
        if body.startswith("Function Name:"):
            cur = body.split(":", 1)[1].strip()
            out[cur] = {}
        elif cur and ":" in body:
            key, val = body.rsplit(":", 1)
            try:
                out[cur][key.strip()] = int(val.strip())
            except ValueError:
                pass
    return out


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source and link the shared library. Returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        return src, _run([cc, *COMMON_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj])

    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(compile_one, zip(srcs, objs)))
    failed = False
    resources = {}
    for src, (rc, out) in results:
        resources.update(parse_resource_usage(out))
        shown = "\n".join(ln for ln in out.splitlines() if "kernel-resource-usage" not in ln)
        if shown.strip() and (verbose or rc != 0):
            print(f"[{os.path.basename(src)}]\n{shown}", file=sys.stderr)
        failed |= rc != 0
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = LIB_PATH + ".tmp"
    rc, out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB_PATH)
    import json
    with open(RESOURCES_PATH, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


# Host-side sanitizers for the ABI check: on hipcc lines each flag follows
# -Xarch_host, so the device code is built as usual.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_CHECK_SRC = os.path.join(ROOT, "tests", "host_check", "abi_host_check.cpp")
HOST_CHECK_EXE = os.path.join(BUILD_DIR, "abi_host_check")


def build_host_check(verbose: bool = False) -> str:
    """Build the ABI host check: api.hip with AddressSanitizer and
    UndefinedBehaviorSanitizer on its host code, the other sources as usual,
    and the checking program tests/host_check/abi_host_check.cpp, linked into one
    executable. Returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, "san_" + os.path.basename(src) + ".o")
        extra = SANITIZE_HOST if os.path.basename(src) == "api.hip" else []
        rc, out = _run([cc, *COMMON_FLAGS, *extra, "-g", "-c", src, "-o", obj])
        if rc != 0:
            print(out, file=sys.stderr)
            raise RuntimeError(f"compiling {src} for the host check failed")
        objs.append(obj)
    drv = os.path.join(BUILD_DIR, "abi_host_check.o")
    gxx = shutil.which("g++") or "g++"
    rc, out = _run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    f"-I{INCLUDE}", "-c", HOST_CHECK_SRC, "-o", drv])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("compiling the host check driver failed")
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(cc))), "lib")
    rc, out = _run([gxx, "-fsanitize=address,undefined", drv, *objs, f"-L{rocm_lib}", "-lamdhip64",
                    f"-Wl,-rpath,{rocm_lib}", "-o", HOST_CHECK_EXE])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("linking the host check failed")
    if verbose:
        print(f"built {HOST_CHECK_EXE}")
    return HOST_CHECK_EXE


if __name__ == "__main__":
    build(verbose=True)
    if len(sys.argv) > 1 and sys.argv[1] == "host-check":
        build_host_check(verbose=True)

"""Build the HIP library of the LSH-attention forward for gfx950 (MI355X).

    python -m lsh_attention_02_amd.build          # or: from lsh_attention_02_amd.build import build
    python -m lsh_attention_02_amd.build --debug  # the same with device-side bounds checks

Compiles every csrc/*.hip with hipcc (in parallel) and links
lsh_attention_02_amd/liblsh_attention.so in-tree.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "liblsh_attention.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
DEBUG_LIB_PATH = os.path.join(PKG, "liblsh_attention_debug.so")
DEBUG_BUILD_DIR = os.path.join(PKG, "_build", "debug")
ARCH = "gfx950"

CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed FP32 instructions are disabled for all device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# MFMA results in ordinary VGPRs: the attention kernel reads its score and
# output accumulators with VALU instructions, and accumulation registers would
# add a copy per value.  Not for the backward, whose live set exceeds the 256
# ordinary VGPRs (its key-gradient accumulators live in accumulation registers),
# nor for the 256 x 256 GEMM tiles (256 accumulators per lane).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
NO_VGPR_FORM = {"lsh_attn_bwd.hip", "lsh_gemm256.hip"}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the LSH-attention library)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [l for l in p.stdout.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l]
    return p.returncode, "\n".join(lines)


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile and link the library; returns its path.  Raises on failure.

    debug: the same library with the device-side bounds checks compiled in
    (LSH_DEVICE_CHECKS; lsh_debug_check_failures reads their counters), as
    DEBUG_LIB_PATH.  The kernels are otherwise the same."""
    cc = hipcc()
    bdir = DEBUG_BUILD_DIR if debug else BUILD_DIR
    os.makedirs(bdir, exist_ok=True)
    sources = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(bdir, s[:-4] + ".o") for s in sources]
    extra = ["-DLSH_DEVICE_CHECKS"] if debug else []
    jobs = [[cc, *CXXFLAGS, *extra, *([] if s in NO_VGPR_FORM else VGPR_FORM), "-c",
             os.path.join(CSRC, s), "-o", o] for s, o in zip(sources, objs)]
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_run, jobs))
    for src, (rc, out) in zip(sources, results):
        if verbose or rc:
            print(f"[build] {src}\n{out}", file=sys.stderr)
        if rc:
            raise RuntimeError(f"hipcc failed on {src}")
    path = DEBUG_LIB_PATH if debug else LIB_PATH
    tmp = path + ".tmp"
    rc, out = _run([cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    if rc:
        print(out, file=sys.stderr)
        raise RuntimeError("linking the LSH-attention library failed")
    os.replace(tmp, path)
    if not debug:
        build_asan_check(objs, verbose)
    return path


ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_CHECK = os.path.join(ASAN_DIR, "abi_asan_check")


def build_asan_check(objs, verbose: bool = False) -> str:
    """The host-only AddressSanitizer check of the C ABI's argument validation
    (tests/abi_asan_check.c, run by tests/test_abi.py): lsh_api.hip's host code
    compiled with ASan (device code untouched), linked with the other objects
    of the library build.  Not part of the library."""
    rocm = os.path.realpath(os.path.join(os.path.dirname(os.path.realpath(hipcc())), ".."))
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    clangxx = clang + "++"
    rocm_inc = os.path.join(rocm, "include")
    rocm_lib = os.path.join(rocm, "lib")
    driver = os.path.join(ROOT, "tests", "abi_asan_check.c")
    os.makedirs(ASAN_DIR, exist_ok=True)
    api_o = os.path.join(ASAN_DIR, "lsh_api.o")
    drv_o = os.path.join(ASAN_DIR, "abi_asan_check.o")
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in CXXFLAGS if f != "-O3"] + ["-O1", "-g"]
    steps = [
        [hipcc(), *flags, *VGPR_FORM, *host_asan, "-c", os.path.join(CSRC, "lsh_api.hip"), "-o", api_o],
        [clang, "-std=c99", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-Wall",
         "-D__HIP_PLATFORM_AMD__", f"-I{rocm_inc}", f"-I{INCLUDE}", "-c", driver, "-o", drv_o],
        [clangxx, "-fsanitize=address", drv_o, api_o,
         *[o for o in objs if os.path.basename(o) != "lsh_api.o"],
         f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{rocm_lib}", "-o", ASAN_CHECK],
    ]
    for cmd in steps:
        rc, out = _run(cmd)
        if verbose or rc:
            print(f"[build] {' '.join(cmd[:3])} ...\n{out}", file=sys.stderr)
        if rc:
            raise RuntimeError("building the ASan check of the C ABI failed")
    return ASAN_CHECK


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv))

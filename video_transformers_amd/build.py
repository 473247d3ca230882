"""Builds libpsa.so (the HIP kernels for gfx950 plus the C ABI host code) in-tree.

    python -m video_transformers_amd.build [-v]

Each source is compiled to an object under _build/ in parallel, then linked into
video_transformers_amd/libpsa.so. hipcc cross-compiles for gfx950 without a GPU present.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpsa.so")

SOURCES = ["psa_api.cpp", "psa_pyramid.hip", "psa_index.hip", "psa_attn.hip", "psa_attn_bf16.hip",
           "psa_attn_bwd.hip", "psa_mask.hip", "psa_fp8.hip"]
HEADERS = ["psa_internal.h", "psa_device.h", "psa_attn_common.h", "psa_bf16_tile.h", "psa_assign.h"]

ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for every device compile: the compiler then never
# emits v_pk_{add,mul,fma}_f32 from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-result"] + DEVICE_FLAGS
# Per-source extras. The bf16 attention and mask-scoring kernels keep their MFMA accumulators
# in VGPRs (the softmax work reads them with VALU instructions; from AGPRs each value would
# first need a v_accvgpr_read). Both are compiled without NaN semantics so that max reductions of MFMA results need no
# canonicalisation (they mask with -inf, never with NaN; infinities keep their meaning), and so that
# the threshold assignment they share (psa_assign.h) compiles to the same arithmetic in both.
EXTRA = {
    "psa_attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
    "psa_mask.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = os.path.join(rocm, "bin", "hipcc")
    if not os.path.exists(exe):
        exe = shutil.which("hipcc") or exe
    return exe


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + CFLAGS + EXTRA.get(src, [])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


# A second build of the host side of the C ABI (psa_api.cpp: argument checks, workspace
# layout, dispatch) with AddressSanitizer and UndefinedBehaviorSanitizer on the host code only,
# linked with the same device objects into _build/libpsa_hostsan.so. The CPU tests run the
# argument checks against it (no GPU needed). Device code is never built with a sanitizer.
HOSTSAN_LIB = os.path.join(BUILD, "libpsa_hostsan.so")
HOSTSAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime the host-sanitized library links against."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    base = os.path.join(rocm, "llvm", "lib", "clang")
    for ver in sorted(os.listdir(base), reverse=True) if os.path.isdir(base) else []:
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise FileNotFoundError("clang AddressSanitizer runtime not found under " + base)


def build_host_sanitized(verbose: bool = False, objs=None) -> str:
    """Compile psa_api.cpp with host sanitizers and link _build/libpsa_hostsan.so with the other
    objects of the last build (compiling them first if absent)."""
    os.makedirs(BUILD, exist_ok=True)
    if objs is None:
        objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        if not all(os.path.exists(o) for o in objs):
            build(verbose)
    obj = os.path.join(BUILD, "psa_api_hostsan.o")
    cmd = ([hipcc(), "-x", "hip", "-c", os.path.join(CSRC, "psa_api.cpp"), "-o", obj, "-g"] +
           [f for f in CFLAGS if f != "-O3"] + ["-O1"] + HOSTSAN_FLAGS)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on psa_api.cpp (host sanitizers):\n{r.stdout}\n{r.stderr}")
    others = [o for o in objs if not o.endswith("psa_api.o")]
    cmd = ([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-shared-libasan", "-o",
            HOSTSAN_LIB + ".tmp", obj] + others + HOSTSAN_FLAGS[:4])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (host sanitizers):\n{r.stdout}\n{r.stderr}")
    os.replace(HOSTSAN_LIB + ".tmp", HOSTSAN_LIB)
    return HOSTSAN_LIB


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source and link libpsa.so (and the host-sanitized build of the C ABI's
    host side). Always recompiles. Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_host_sanitized(verbose, objs)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))

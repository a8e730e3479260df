"""Build the gfx950 HIP library ``libfa.so`` in-tree with hipcc.

Usage: ``python -m exact_io_aware_29_amd.build`` (or ``build()`` from Python).
Every source is compiled for gfx950 only; packed-fp32 instructions are
disabled for all device code.
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
OUT = os.path.join(PKG, "libfa.so")
OBJDIR = os.path.join(ROOT, "_build")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_bwd.hip", "fa_decode.hip",
           "fa_scratch.hip"]
# Per-source extra flags. Matrix-core results go to VGPRs (the softmax reads
# them directly, without v_accvgpr_read); the register allocator then uses
# AGPRs as overflow for long-lived values.
EXTRA = {"fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


# Kernel sources only: the kernels never produce NaN from valid input, which
# lets fmaxf lower to a bare v_max_f32 (infinities keep their IEEE meaning).
# The host-side API validates user floats and must see NaN as NaN.
KERNEL_FLAGS = ["-fno-honor-nans"]


# The debug variant: a workgroup barrier before every refill of an LDS stage
# and a full wait plus barrier right after it (FA_PARANOID_BARRIERS in
# fa_stage.h). Its results must equal the release library's bit for bit;
# the GPU tests compare the two. Nothing else loads it.
PARANOID_OUT = os.path.join(PKG, "libfa_paranoid.so")
PARANOID_FLAGS = ["-DFA_PARANOID_BARRIERS=1"]


# Debug variant with per-workgroup timelines (FA_TIMELINE in fa_device.h):
# the 16x16x32 forward, dQ and dK/dV kernels stamp entry, block, first-tile,
# loop-end and exit times into device arrays that `bench.py --timeline`
# reads (include/fa_timeline.h). Nothing else loads it.
TIMELINE_OUT = os.path.join(PKG, "libfa_timeline.so")
TIMELINE_FLAGS = ["-DFA_TIMELINE=1"]


# Measurement only: the instruction-mix ceiling of the matrix-core kernels
# (a grid of products / exponentials / other VALU mixes, timed by
# ``bench.py --mix-ceiling``). The attention library does not load it.
MIXBENCH_SRC = "mixbench.hip"
MIXBENCH_OUT = os.path.join(PKG, "libfa_mixbench.so")


def _compile(job) -> str:
    src, variant = job
    if variant == "mixbench":
        tmp = MIXBENCH_OUT + ".tmp"
        cmd = [HIPCC, *FLAGS, "-shared", "-x", "hip", os.path.join(CSRC, src), "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, MIXBENCH_OUT)
        return MIXBENCH_OUT
    objdir = os.path.join(OBJDIR, variant) if variant else OBJDIR
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip", *KERNEL_FLAGS] if src.endswith(".hip") else []
    extra = {"paranoid": PARANOID_FLAGS, "timeline": TIMELINE_FLAGS}.get(variant, [])
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *extra, *lang, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


# Host-sanitizer build of the C ABI layer, for the CPU tests: fa_api.cpp (all
# host code: argument checks and launches) compiled by g++ with AddressSanitizer
# and UndefinedBehaviorSanitizer, linked with the release kernel objects. The
# CPU test suite loads it (FA_LIBRARY) with the sanitizer runtime preloaded.
SANITIZED_OUT = os.path.join(OBJDIR, "libfa_sanitized.so")
ASAN_RUNTIME = "/usr/lib/x86_64-linux-gnu/libasan.so.6"
_SAN = "-fsanitize=address,undefined"


def build_sanitized(verbose: bool = False):
    """Build SANITIZED_OUT from the release objects (call after build());
    returns its path, or None when g++ or the sanitizer runtime is absent."""
    if shutil.which("g++") is None or not os.path.exists(ASAN_RUNTIME):
        return None
    obj = os.path.join(OBJDIR, "fa_api_sanitized.o")
    cc = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", _SAN,
          "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
          "-c", os.path.join(CSRC, "fa_api.cpp"), "-o", obj]
    kernels = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o")
               for s in SOURCES if s != "fa_api.cpp"]
    ld = ["g++", "-shared", _SAN, obj, *kernels, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", SANITIZED_OUT]
    for cmd in (cc, ld):
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized build failed:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SANITIZED_OUT}")
    return SANITIZED_OUT


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libfa.so``, the debug variants
    ``libfa_paranoid.so`` and ``libfa_timeline.so`` and the measurement
    library ``libfa_mixbench.so``; returns the path of ``libfa.so``."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(os.path.join(OBJDIR, "paranoid"), exist_ok=True)
    os.makedirs(os.path.join(OBJDIR, "timeline"), exist_ok=True)
    n = len(SOURCES)
    jobs = ([(s, "") for s in SOURCES] + [(s, "paranoid") for s in SOURCES] +
            [(s, "timeline") for s in SOURCES] + [(MIXBENCH_SRC, "mixbench")])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:n], OUT)
    _link(objs[n:2 * n], PARANOID_OUT)
    _link(objs[2 * n:3 * n], TIMELINE_OUT)
    if verbose:
        print(f"built {OUT}, {PARANOID_OUT}, {TIMELINE_OUT} and {MIXBENCH_OUT}")
    build_sanitized(verbose)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

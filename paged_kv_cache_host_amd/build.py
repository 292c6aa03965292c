"""Build libpa.so (host allocator + HIP kernels for gfx950) in-tree.

    python -m paged_kv_cache_host_amd.build          # or build() from Python

Every source is compiled with hipcc for gfx950 only.  Packed-fp32 VALU
instructions are disabled on the device side (-packed-fp32-ops) so that
float code is never lowered to them.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpa.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["pa_host.cpp", "pa_sched.cpp", "pa_timing.cpp", "pa_cache_write.hip", "pa_decode.hip", "pa_generic.hip", "pa_prefill.hip", "pa_stage.hip", "pa_varlen.hip", "pa_decode_step.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm is required to build libpa)")
    return p


def _flags(src: str) -> list[str]:
    f = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-I", INCLUDE, "-I", CSRC]
    if src.endswith(".hip"):
        f += ["-x", "hip", f"--offload-arch={ARCH}",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-fno-gpu-rdc"]
    return f


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *_flags(src), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        msg = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
        if msg.strip():
            print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host code of the library (allocator, scheduler, timing) built with
# AddressSanitizer and UndefinedBehaviorSanitizer by the ROCm clang for the
# host only, linked with the kernels' objects of the last build() (device
# code unsanitised).  The CPU parity tests of the host code run against it
# with PA_LIBRARY set to its path and the clang sanitizer runtime preloaded.
SANITIZED_SOURCES = ["pa_host.cpp", "pa_sched.cpp", "pa_timing.cpp"]
SANITIZE = ["-fsanitize=address,undefined", "-shared-libasan", "-fno-omit-frame-pointer"]


def host_clang() -> str:
    p = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang++")
    p = os.path.normpath(p)
    if not os.path.exists(p):
        p = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(p):
        raise RuntimeError("the ROCm clang++ is required for the sanitizer build")
    return p


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime to preload into Python."""
    r = subprocess.run([host_clang(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return r.stdout.strip()


def build_sanitized(out_dir: str | None = None, verbose: bool = False) -> str:
    out_dir = out_dir or os.path.join(BUILD_DIR, "sanitized")
    os.makedirs(out_dir, exist_ok=True)
    kernels = [os.path.join(BUILD_DIR, s + ".o") for s in SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(k) for k in kernels):
        build(verbose)
    cxx = host_clang()
    objs = []
    for src in SANITIZED_SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        cmd = [cxx, "-std=c++17", "-O1", "-g", "-fPIC", *SANITIZE, "-D__HIP_PLATFORM_AMD__",
               "-I", os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "include"),
               "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    lib = os.path.join(out_dir, "libpa_sanitized.so")
    rocm_lib = os.path.normpath(os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..",
                                             "lib"))
    cmd = [cxx, "-shared", *SANITIZE, "-o", lib, *objs, *kernels, "-L", rocm_lib,
           "-lamdhip64", f"-Wl,-rpath,{rocm_lib}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)

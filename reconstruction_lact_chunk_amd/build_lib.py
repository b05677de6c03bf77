"""Build the HIP library libzmttt.so in-tree with hipcc for gfx950.

Usage: python -m reconstruction_lact_chunk_amd.build_lib [--verbose]
Objects go to _build/ at the repository root; the shared library lands next
to this file, where the Python binding loads it from.
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
LIB = os.path.join(PKG, "libzmttt.so")
ARCH = "gfx950"

SOURCES = ["weights.hip", "update_bf16.hip", "apply_bf16.hip", "frame_bf16.hip", "fp32_path.hip",
           "newton_schulz.hip", "wide_kernels.hip", "wide_gemm.hip", "wide_path.cpp", "gemm_lt.cpp",
           "layer_kernels.hip", "wide_ns.hip", "api.cpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Packed fp32 VALU forms are kept out of the generated code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Address and undefined-behaviour sanitizers for the host half only (argument
# validation, workspace carving, launch set-up); device code is built as usual.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _compile(src: str, verbose: bool, defines=(), build_dir=BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    defs = [f"-D{d}" for d in defines]
    cmd = [hipcc(), *COMMON, *defs, *DEVICE, *extra, "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, flush=True)
    return obj


def build(verbose: bool = False, defines=(), out: str = LIB, host_sanitize: bool = False) -> str:
    """Compile every source and link the library (default: libzmttt.so next
    to this file); `defines` are extra preprocessor definitions such as tuning
    switches.  host_sanitize instruments the host code with ASan and UBSan (the
    resulting library needs the sanitizer runtime preloaded; see
    sanitizer_runtime()).  Returns the library path."""
    if host_sanitize and out == LIB:
        raise ValueError("a sanitized build goes to its own path, not over the product library")
    build_dir = BUILD if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    extra = HOST_SANITIZE if host_sanitize else ()
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, defines, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "lib")
    # hipBLASLt serves the plain GEMMs of the full-width head shape
    cmd = [hipcc(), *DEVICE, "-shared", "-fPIC", "-o", tmp, *objs, f"-L{rocm_lib}", "-lhipblaslt",
           f"-Wl,-rpath,{rocm_lib}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


def sanitizer_runtime() -> str:
    """Path of the compiler's shared ASan runtime (it carries the UBSan
    handlers too), to be preloaded into a process that loads a sanitized
    build."""
    res = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm",
                                       "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("shared ASan runtime not found")
    return path


if __name__ == "__main__":
    defs = [a[2:] for a in sys.argv[1:] if a.startswith("-D")]
    outs = [a.split("=", 1)[1] for a in sys.argv[1:] if a.startswith("--out=")]
    print(build(verbose="--verbose" in sys.argv, defines=defs, out=outs[0] if outs else LIB))

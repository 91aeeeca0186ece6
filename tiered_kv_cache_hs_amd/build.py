"""Build libhisparse.so for gfx950 with hipcc (in-tree, next to this file).

    python -m tiered_kv_cache_hs_amd.build

Every HIP source is compiled with packed-fp32 instruction selection turned
off (-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass warns
that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libhisparse.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["runtime.hip", "resolve.hip", "attn_mha.hip", "attn_latent.hip", "stage.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source additions. The latent attention kernel assumes no NaN operands
# (its error outputs are written as NaN bit patterns), which lets max and its
# DPP lane moves compile to single v_max_f32_dpp instructions.
EXTRA = {"attn_latent.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}


# Host-code sanitizers for a CPU-only test build (build_host_sanitized): each
# flag applies to the host pass only; the device code is built as always.
HOST_SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all",
                  "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, objdir: str = OBJDIR, extra=()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # drop the host pass's notice about the device-only feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link libhisparse.so. Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_host_sanitized(out: str) -> str:
    """The library with AddressSanitizer and UndefinedBehaviorSanitizer on its
    host code (argument checks, handles, planning), for CPU tests in a process
    that preloads the sanitizer runtime: out/libhisparse_san.so."""
    objdir = os.path.join(out, "obj")
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir, HOST_SAN_FLAGS), SOURCES))
    lib = os.path.join(out, "libhisparse_san.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    build()

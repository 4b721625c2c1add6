"""Builds libaut.so (HIP kernels for gfx950 + the C-ABI host layer) in-tree.

    python -m packed_windowed_attention_amd.build

Each source is compiled by hipcc into _build/ at the repository root, then
linked into packed_windowed_attention_amd/libaut.so (written to a temporary
name and renamed, so a concurrent loader never sees half a file).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libaut.so")

SOURCES = ["aut_host.cpp", "k_stem.hip", "k_gemm128.hip", "k_gemm256.hip", "k_ln.hip", "k_attn.hip", "k_inject.hip",
           "k_logmel.hip", "k_mx.hip", "k_scratch.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed fp32 arithmetic is switched off for the device code: the compiler
# still emits scalar or vector fp32 math, never the packed forms.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function", f"-I{ROOT}/include"]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _check_launch_stubs(lib: str) -> None:
    """Every kernel the host code launches has its launch stub in the library.
    (The host compilation pass can leave a kernel template's stubs undefined
    without a diagnostic; the library would then fail only when loaded.)"""
    r = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"nm failed on {lib}:\n{r.stderr}")
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        os.unlink(lib)
        raise RuntimeError("kernel launch stubs missing from the library: " + ", ".join(missing[:8]))


def build(verbose: bool = False) -> str:
    """Compiles every source and links libaut.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    workers = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    _check_launch_stubs(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)

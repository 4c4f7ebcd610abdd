"""Builds libmla.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Usage: python -m mla_latent_kv_27_amd.build [--variant release|debug|asan]  (or call build()).
Compiles every time it is called; objects go to mla_latent_kv_27_amd/_build/, the libraries to
mla_latent_kv_27_amd/lib/: libmla.so (the MLA kernels and the C ABI) and libmla_probe.so (the HBM
streaming-ceiling probe the benchmark reports against; no part of the MLA computation).

Variants, each its own library beside the release one (select it with the MLA_LIBRARY
environment variable; the binding loads libmla.so otherwise):
  debug  libmla_debug.so: built with MLA_DEBUG, the host checks the block ids and context lengths
         it reads from device memory before launching, and synchronises after every launch group;
  asan   libmla_asan.so: the host code under AddressSanitizer and UndefinedBehaviorSanitizer (the
         device code is unchanged); load it with the sanitizer runtime preloaded, on the CPU (the
         tests run the host-side C ABI checks with it).
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
LIB = os.path.join(PKG, "lib", "libmla.so")
PROBE_LIB = os.path.join(PKG, "lib", "libmla_probe.so")
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["gemm.hip", "rope.hip", "decode_attn.hip", "prefill_attn.hip", "latent_fp8.hip", "mla_api.cpp"]
PROBE_SOURCES = ["probe.hip"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 ALU forms stay off: the compiler emits plain fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # the decode kernel sets M0 (the LDS destination of its copies) inside one asm statement
    "-Wno-inline-asm",
]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmla)")


VARIANTS = {
    "release": ([], [], LIB),
    "debug": (["-DMLA_DEBUG"], [], os.path.join(PKG, "lib", "libmla_debug.so")),
    # host code only: each sanitizer flag goes to the host compilation
    "asan": (["-g", "-Xarch_host", "-fno-omit-frame-pointer",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=undefined"],
             ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"],
             os.path.join(PKG, "lib", "libmla_asan.so")),
}


def _compile(src, extra=(), sub=""):
    os.makedirs(os.path.join(BUILD, sub), exist_ok=True)
    obj = os.path.join(BUILD, sub, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *extra, "-I", INCLUDE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out, extra=()):
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(out)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, variant: str = "release") -> str:
    """Builds the library of `variant` (and, for release, the probe library); returns its path."""
    cflags, lflags, out = VARIANTS[variant]
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    srcs = SOURCES + (PROBE_SOURCES if variant == "release" else [])
    sub = "" if variant == "release" else variant
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, cflags, sub), srcs))
    _link(objs[:len(SOURCES)], out, lflags)
    if variant == "release":
        _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", out, *(["and", PROBE_LIB] if variant == "release" else []))
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--variant", choices=sorted(VARIANTS), default="release")
    build(verbose=True, variant=ap.parse_args().variant)

"""Build libgdr.so (the HIP kernels and C-ABI entry points) for gfx950, in-tree.

Each ``csrc/*.hip`` file is compiled to an object with hipcc in parallel and
linked into ``matrix_memory_rnn_amd/libgdr.so``. Packed-fp32 VALU forms are
disabled for device code (``-packed-fp32-ops``); hipcc's host pass warns that it
does not know that feature, which is harmless.

Two more libraries share the kernel objects and differ only in the entry-point
sources (``DEBUG_SOURCES``):

- ``libgdr_debug.so``: compiled with ``GDR_DEBUG`` defined, so every entry
  point checks its inputs' values on the GPU before its compute kernels;
- ``libgdr_hostsan.so``: the entry points' host code instrumented with
  AddressSanitizer and UndefinedBehaviorSanitizer (host code only: the device
  code is built as usual). It is loaded only by a CPU test that preloads the
  sanitizer runtime and drives the argument-validation paths.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdr.so")
LIB_DEBUG = os.path.join(PKG, "libgdr_debug.so")
LIB_HOSTSAN = os.path.join(PKG, "libgdr_hostsan.so")
# the sources that differ between the three libraries
DEBUG_SOURCES = ("gdr_api.hip", "gdr_debug.hip")
HOSTSAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]
ARCH = os.environ.get("GDR_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-result",
]


def _compile(job) -> str:
    src, variant = job
    out_dir = BUILD if variant == "release" else os.path.join(BUILD, variant)
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    extra = {"release": [], "debug": ["-DGDR_DEBUG"], "hostsan": HOSTSAN_FLAGS}[variant]
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src} ({variant}):\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib, extra=()):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libgdr.so, libgdr_debug.so and
    libgdr_hostsan.so; returns the path of libgdr.so."""
    for d in (BUILD, os.path.join(BUILD, "debug"), os.path.join(BUILD, "hostsan")):
        os.makedirs(d, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    special = [s for s in srcs if os.path.basename(s) in DEBUG_SOURCES]
    jobs_list = [(s, "release") for s in srcs] + [(s, v) for v in ("debug", "hostsan") for s in special]
    jobs = min(len(jobs_list), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = dict(zip(jobs_list, ex.map(_compile, jobs_list)))
    release = [objs[(s, "release")] for s in srcs]
    _link(release, LIB)
    for variant, lib, extra in (("debug", LIB_DEBUG, ()),
                                ("hostsan", LIB_HOSTSAN, ("-Xarch_host", "-fsanitize=address", "-Xarch_host",
                                                          "-fsanitize=undefined", "-shared-libsan"))):
        _link([objs[(s, variant if s in special else "release")] for s in srcs], lib, extra)
    if verbose:
        print(f"built {LIB}, {LIB_DEBUG}, {LIB_HOSTSAN}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

"""Build libbitdelta.so for gfx950 with hipcc, in-tree.

Every HIP source compiles for gfx950 only, with packed-fp32 instruction
selection disabled (the kernels never rely on v_pk_*_f32).
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libbitdelta.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

SOURCES = ["api.cpp", "cache.cpp", "compress.hip", "decode.hip", "shot.hip", "slice.hip", "gemv.hip", "quad.hip", "band.hip", "skinny.hip", "rowstream.hip", "prefill.hip",
           "grouped.hip", "gdec.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + INCLUDE, "-I" + CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


PROBE_SOURCE = os.path.join(CSRC, "probe", "stream_read.hip")
PROBE_LIBRARY = os.path.join(PKG, "libbdprobe.so")


def build_probe(verbose: bool = False) -> str:
    """The benchmark's stream-read probe (not part of libbitdelta)."""
    tmp = PROBE_LIBRARY + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-shared", PROBE_SOURCE, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the probe:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, PROBE_LIBRARY)
    if verbose:
        print("built", PROBE_LIBRARY)
    return PROBE_LIBRARY


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link libbitdelta.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIBRARY)
    if verbose:
        print("built", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    build_probe(verbose=True)

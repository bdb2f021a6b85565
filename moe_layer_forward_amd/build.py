"""In-tree build of the native libraries (gfx950 HIP code and the host-side generator).

    python -m moe_layer_forward_amd.build

compiles, next to their sources:

* ``libmoe.so``           -- the MoE layer kernels behind the C ABI of ``include/moe.h``;
* ``libmoe_peaks.so``     -- measured machine peaks (streaming read, copy, MFMA loop) for the benchmark;
* ``synth/libsynth_dev.so``  -- device side of the seeded input generator;
* ``synth/libsynth_host.so`` -- host side of the seeded input generator (gcc, OpenMP).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SYNTH = os.path.join(PKG, "synth")
INCLUDE = os.path.join(ROOT, "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

MOE_SOURCES = ["moe_api.cpp", "route.hip", "permute.hip", "gemm_stream.hip", "gemm_tile.hip", "gemm_tile_q4.hip",
               "gemm_skinny.hip",
               "gemm_quant.hip", "gemm_simple.hip", "combine.hip"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build failed: {' '.join(cmd[:3])} ...")
    return r


def build_synth_host(verbose=False):
    out = os.path.join(SYNTH, "libsynth_host.so")
    _run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", out,
          os.path.join(SYNTH, "synth_host.c"), "-lm"], verbose)
    return out


def build_synth_dev(verbose=False):
    out = os.path.join(SYNTH, "libsynth_dev.so")
    _run([HIPCC, *HIP_FLAGS, "-o", out, os.path.join(SYNTH, "synth_dev.hip")], verbose)
    return out


def build_moe(verbose=False, jobs=None):
    """libmoe.so: every source compiled to an object in parallel (one hipcc process each, at most
    `jobs` at a time), then linked."""
    out = os.path.join(PKG, "libmoe.so")
    objdir = tempfile.mkdtemp(prefix="moe_objs_")
    try:
        def compile_one(name):
            obj = os.path.join(objdir, os.path.splitext(name)[0] + ".o")
            flags = [f for f in HIP_FLAGS if f != "-shared"]
            _run([HIPCC, *flags, "-c", f"-I{INCLUDE}", f"-I{CSRC}", "-x", "hip", os.path.join(CSRC, name),
                  "-o", obj], verbose)
            return obj

        jobs = jobs or max(1, min(len(MOE_SOURCES), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            objs = list(pool.map(compile_one, MOE_SOURCES))
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out], verbose)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return out


def build_peaks(verbose=False):
    out = os.path.join(PKG, "libmoe_peaks.so")
    _run([HIPCC, *HIP_FLAGS, "-o", out, os.path.join(CSRC, "peaks.hip")], verbose)
    return out


def build_all(verbose=False):
    build_synth_host(verbose)
    build_synth_dev(verbose)
    build_peaks(verbose)
    if all(os.path.exists(os.path.join(CSRC, s)) for s in MOE_SOURCES):
        build_moe(verbose)
    else:
        raise RuntimeError("libmoe sources missing")


if __name__ == "__main__":
    build_all(verbose=True)

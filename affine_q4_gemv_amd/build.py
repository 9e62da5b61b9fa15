"""Build libq4mv.so (gfx950) in-tree with hipcc, and libq4mv_probe.so (the measurement
reference kernels the benchmark times next to the GEMV).

Usage: ``python -m affine_q4_gemv_amd.build`` (or ``build()`` from Python). Each ``.hip``
source is compiled to an object in parallel, then linked into
``affine_q4_gemv_amd/libq4mv.so`` (sources in ``csrc/``) and
``affine_q4_gemv_amd/libq4mv_probe.so`` (sources in ``csrc/probe/``).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq4mv.so")
LIB_PROBE = os.path.join(HERE, "libq4mv_probe.so")
BUILD_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",                     # only the fmas written in the source
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",  # no v_pk_*_f32
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def probe_sources():
    return sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], check=True,
                   stderr=subprocess.PIPE if os.environ.get("Q4MV_QUIET") else None)
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, lib)


def build(jobs: int | None = None) -> str:
    """Compile every HIP source for gfx950 and link libq4mv.so and libq4mv_probe.so.
    Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    probes = probe_sources()
    with cf.ThreadPoolExecutor(max_workers=jobs or min(8, len(srcs) + len(probes))) as ex:
        objs = list(ex.map(_compile, srcs + probes))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], LIB_PROBE)
    return LIB


if __name__ == "__main__":
    print(build())

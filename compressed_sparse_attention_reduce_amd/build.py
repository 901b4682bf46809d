"""Ahead-of-time build of libcsa.so (the C-ABI library) for gfx950.

Every ``csrc/*.hip`` file is compiled with hipcc to an object in ``_build/``
(in parallel), then linked into ``libcsa.so`` next to this file; the
calibration probes in ``csrc/calib/`` go into ``libcsa_calib.so`` beside it
(include/csa_calib.h).  All device code is built with packed-FP32
instruction selection disabled.
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
LIB = os.path.join(PKG, "libcsa.so")
CALIB_LIB = os.path.join(PKG, "libcsa_calib.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int = 8) -> str:
    """Compile every HIP source and link libcsa.so and libcsa_calib.so;
    returns the path of libcsa.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    calib_dir = os.path.join(CSRC, "calib")
    calib = sorted(os.path.join(calib_dir, f) for f in os.listdir(calib_dir) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs) + len(calib)))) as ex:
        objs = list(ex.map(_compile, srcs + calib))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], CALIB_LIB)
    return LIB


if __name__ == "__main__":
    print(build())

"""Build libsinkattn.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950.

    python -m sliding_window_sink_amd.build        # compile every source, link

Each ``csrc/*.hip`` is compiled to an object in parallel, then linked into
``sliding_window_sink_amd/libsinkattn.so`` next to this file.  The build always
recompiles (it is the "does it build" check); loading the library never builds.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsinkattn.so")
# calibration kernels of the benchmark's measured ceilings (not the attention path)
CALIB_SRC = os.path.join(HERE, "calib", "stream_read.hip")
CALIB_LIB = os.path.join(HERE, "libsinkattn_calib.so")
ARCH = os.environ.get("SINKATTN_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops (v_pk_*_f32) are turned off: plain fp32 code only.
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(HERE, "..", "include"), "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources) + 1)) as ex:
        calib = ex.submit(_compile, CALIB_SRC)
        objs = list(ex.map(_compile, sources))
        calib_obj = calib.result()
    _link(objs, LIB)
    _link([calib_obj], CALIB_LIB)
    if verbose:
        print("built", LIB, "and", CALIB_LIB)
    return LIB


if __name__ == "__main__":
    build()

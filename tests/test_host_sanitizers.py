"""The C ABI's host validation layer under AddressSanitizer and UBSan (CPU only).

``csrc/api.hip`` (argument checks, split-K planning, alias checks, status codes)
is built with its host half instrumented (``-Xarch_host -fsanitize=...``: the
device half is never instrumented) and linked with stub launchers that record
each launch instead of running a kernel.  A driver then calls every entry point
with valid and invalid arguments, passing host buffers of exactly the
documented tensor sizes in place of device pointers, and checks every status
code and the recorded launch parameters.  A second run makes a deliberate
one-byte heap overread to show that the sanitizer is active in the build.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_asan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer"] + SAN + \
    ["-Xarch_host", "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include")]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("host_asan")
    objs = []
    jobs = [(os.path.join(ROOT, "sliding_window_sink_amd", "csrc", "api.hip"),
             ["-x", "hip", "--offload-arch=gfx950"]),
            (os.path.join(HERE, "stub_launchers.cpp"), ["-x", "hip", "--offload-host-only"]),
            (os.path.join(HERE, "driver.cpp"), ["-x", "hip", "--offload-host-only"])]
    for src, mode in jobs:
        obj = str(out / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC] + mode + FLAGS + ["-c", src, "-o", obj], capture_output=True,
                           text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(out / "driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950"] + SAN + objs + ["-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    yield exe
    shutil.rmtree(str(out), ignore_errors=True)


def test_validation_layer_is_clean_under_sanitizers(driver):
    r = subprocess.run([driver], capture_output=True, text=True, timeout=120, env=ENV)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert " 0 failed" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_sanitizer_is_live(driver):
    r = subprocess.run([driver, "selfcheck"], capture_output=True, text=True, timeout=120, env=ENV)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr

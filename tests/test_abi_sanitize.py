"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

abi.hip and calib.hip (every exported entry point and its validation) are
compiled with the sanitizers on their host side only; the device code and the other objects are
the ordinary build. tests/abi_checks.c calls every entry point with invalid
and extreme arguments that the library rejects before any HIP call, so the
run needs no GPU and launches nothing. Any sanitizer report, or a return code
other than the documented one, fails the test.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from int4_weight_only_moe_amd import build as b

SAN_DIR = os.path.join(b.BUILD, "san")
SANITIZED = ("abi.hip", "calib.hip")  # the sources holding the exported entry points
CLANG = "/opt/rocm/llvm/bin/clang"
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


def _objects():
    """Ordinary objects of every source but the sanitized ones (compiled if missing or stale)."""
    objs = []
    for src in b.sources():
        if os.path.basename(src) in SANITIZED:
            continue
        obj = os.path.join(b.BUILD, os.path.basename(src)[:-4] + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(src):
            os.makedirs(b.BUILD, exist_ok=True)
            obj = b._compile(src)
        objs.append(obj)
    return objs


@pytest.fixture(scope="module")
def checker():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("host-only check: its calls pass host pointers, so it runs where no GPU is visible")
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang not found")
    os.makedirs(SAN_DIR, exist_ok=True)
    san_objs = []
    for src in SANITIZED:
        obj = os.path.join(SAN_DIR, src[:-4] + ".o")
        _run([b.hipcc(), *b.COMMON, "-O1", "-g", "-fno-omit-frame-pointer", *SANITIZE_HOST, "-c",
              os.path.join(b.CSRC, src), "-o", obj])
        san_objs.append(obj)
    drv_o = os.path.join(SAN_DIR, "abi_checks.o")
    _run([CLANG, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I", os.path.join(b.ROOT, "include"), "-c",
          os.path.join(os.path.dirname(__file__), "abi_checks.c"), "-o", drv_o])
    exe = os.path.join(SAN_DIR, "abi_checks")
    _run([CLANG + "++", "-fsanitize=address,undefined", drv_o, *san_objs, *_objects(), "-L/opt/rocm/lib",
          "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    yield exe
    shutil.rmtree(SAN_DIR, ignore_errors=True)


def test_abi_validation_under_sanitizers(checker):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=24"
    env["HIP_VISIBLE_DEVICES"] = "-1"
    r = subprocess.run([checker], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert "abi checks:" in r.stdout and "passed" in r.stdout

"""The CPU oracle and the C ABI's host-side validation under
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle is built with gcc from oracle.c and a driver that runs every
function on small ragged shapes. The library's sources are compiled for the
host only (no device code; the sanitizers act on host code alone) and linked
with a driver that calls every entry point with invalid arguments and, on a
machine without a GPU, with valid ones that stop at BL_ERR_NO_DEVICE."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_check")
    r = _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
              "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              os.path.join(SAN, "oracle_check.c"), os.path.join(ROOT, "oracle", "oracle.c"),
              "-o", exe, "-lm"])
    assert r.returncode == 0, r.stderr
    r = _run([exe], env=SAN_ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout


def test_abi_host_validation_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    import sys
    sys.path.insert(0, ROOT)
    from ternary_weight_linear_quant_amd import build as blbuild
    # The library's flags without -O3 / -shared / -fPIC; the sanitizers on the
    # host side only.
    flags = [f for f in blbuild.HIP_FLAGS if f not in ("-O3", "-shared", "-fPIC", "-Wall")]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    exe = str(tmp_path / "abi_host_check")
    r = _run([HIPCC, *flags, "-O1", "-g", *san, *blbuild.sources(),
              os.path.join(SAN, "abi_host_check.cpp"), "-o", exe])
    assert r.returncode == 0, r.stderr
    r = _run([exe], env=dict(SAN_ENV, HIP_VISIBLE_DEVICES=""))
    if r.returncode == 77:
        pytest.skip("a GPU is visible")
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout

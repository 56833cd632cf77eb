"""The host side under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host code (packer, validator, padding check, the container
parser that reads untrusted bytes, the head recipe) and the C oracle are each
built into a small driver with -fsanitize=address,undefined and no recovery,
then driven over random valid inputs and truncated or corrupted ones
(tests/sanitize_host.cpp, tests/sanitize_oracle.c). Any out-of-bounds access,
leak or undefined behaviour aborts the driver; a wrong status fails it. The
two are separate executables: the library and the oracle share no code.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_library_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host")
    _run(["g++", "-std=c++17", *SAN, "-I" + os.path.join(ROOT, "include"),
          "-I" + os.path.join(ROOT, "decode_gemv_02_amd", "csrc"), os.path.join(ROOT, "tests", "sanitize_host.cpp"),
          os.path.join(ROOT, "decode_gemv_02_amd", "csrc", "vbq_host.cpp"), "-o", exe], ROOT)
    r = _run([exe, "120"], ROOT)
    assert "0 failures" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle")
    _run(["gcc", "-std=c99", *SAN, "-ffp-contract=off", os.path.join(ROOT, "oracle", "vbq_oracle.c"),
          os.path.join(ROOT, "tests", "sanitize_oracle.c"), "-o", exe, "-lm"], ROOT)
    r = _run([exe, "120"], ROOT)
    assert "0 failures" in r.stdout

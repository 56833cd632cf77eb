"""Compile the VBQ HIP library for gfx950 into decode_gemv_02_amd/libvbq.so."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libvbq.so")
SOURCES = ["vbq_host.cpp", "vbq_device.hip", "vbq_quantize.hip", "vbq_probe.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra",
    "-Wno-unused-parameter", "-fvisibility=hidden",
    # no packed-fp32 VALU ops anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def build(out: str = LIB_PATH, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *sources(), "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())

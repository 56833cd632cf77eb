"""The GEMV, GEMM, unpack and quantizer kernels keep every live value in registers.

A register spill puts a per-lane private segment in HBM: every wave then
writes and re-reads it, which shows up as extra memory traffic of a few KiB
per workgroup. The device code is compiled to gfx950 assembly here (no GPU
needed) and each kernel's private segment size must be zero.
"""
import os
import re
import subprocess

import pytest

from decode_gemv_02_amd import build as B


def _assembly(tmp_path_factory, name):
    out = tmp_path_factory.mktemp("asm") / (name + ".s")
    src = os.path.join(B.CSRC, name)
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", str(out)], check=True,
                   stderr=subprocess.DEVNULL)
    return out.read_text()


@pytest.mark.parametrize("source, kernel_names", [
    ("vbq_device.hip", ("gemv_tiles", "gemv_rows", "gemv_uniform", "unpack_tiles", "gemm_frag")),
    ("vbq_quantize.hip", ("quantize_groups",)),
])
def test_kernels_do_not_spill(tmp_path_factory, source, kernel_names):
    assembly = _assembly(tmp_path_factory, source)
    sizes = dict(re.findall(r"\.set (\S+)\.private_seg_size, (\d+)", assembly))
    kernels = {k: int(v) for k, v in sizes.items() if any(n in k for n in kernel_names)}
    assert kernels, "no kernels found in the assembly"
    assert all(v == 0 for v in kernels.values()), kernels

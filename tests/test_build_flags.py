"""The device code is built without packed-fp32 instructions.

Every HIP source is compiled with ``-Xclang -target-feature -Xclang
-packed-fp32-ops``.  hipcc's host pass warns that it does not know the
feature; the gfx950 pass honours it.  Shown on a small float2 kernel (which
the compiler turns into a packed fused multiply-add without the flag) and
checked on the library's own gfx950 assembly.  CPU only: hipcc
cross-compiles.
"""

import glob
import os
import re
import subprocess

import pytest

from row_wise_top_topk_amd import build as B

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAG = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
PACKED = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")

PROBE = r"""
#include <hip/hip_runtime.h>
__global__ void axpy2(float2* a, const float2* b, float s) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  float2 x = a[i];
  const float2 y = b[i];
  x.x = x.x * s + y.x;
  x.y = x.y * s + y.y;
  a[i] = x;
}
"""

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _device_asm(src, out, flags):
    subprocess.run([HIPCC, "-O3", f"--offload-arch={B.ARCH}", "--cuda-device-only", "-S",
                    *flags, "-o", out, src], check=True, capture_output=True)
    return open(out).read()


def test_flag_removes_packed_fp32_from_device_code(tmp_path):
    src = tmp_path / "probe.hip"
    src.write_text(PROBE)
    without = _device_asm(str(src), str(tmp_path / "without.s"), [])
    with_flag = _device_asm(str(src), str(tmp_path / "with.s"), FLAG)
    assert PACKED.search(without), "the probe no longer shows packed fp32 without the flag"
    assert not PACKED.search(with_flag)


def test_build_passes_the_flag():
    cmd = B.hipcc_command()
    i = cmd.index("-packed-fp32-ops")
    assert cmd[i - 3:i + 1] == FLAG


def test_library_device_code_has_no_packed_fp32(tmp_path):
    out = str(tmp_path / "lib.so")
    cwd = os.getcwd()
    os.chdir(tmp_path)
    try:
        B.build(out, "O3", ["-save-temps=obj"])
    finally:
        os.chdir(cwd)
    asm = [p for p in glob.glob(str(tmp_path / "*.s")) if "gfx950" in p]
    assert asm, "no gfx950 assembly was written"
    for p in asm:
        text = open(p).read()
        assert "v_" in text
        assert not PACKED.search(text), p

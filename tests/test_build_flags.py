"""The library's build flags keep packed fp32 instructions out of gfx950 code.

``build.FLAGS`` turns the ``packed-fp32-ops`` target feature off. hipcc's host
pass does not know the feature and warns about it; this checks that the device
pass honours it: a kernel of float2 multiply-adds compiled with the library's
flags has no packed fp32 instruction in its gfx950 assembly, while the same
kernel built without the feature switch does (the control)."""

import os
import shutil
import subprocess

import pytest

KERNEL = r"""
#include <hip/hip_runtime.h>
__global__ void k(float2* a, const float2* b, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    float2 x = a[i], y = b[i];
    x.x = x.x * y.x + 1.0f;
    x.y = x.y * y.y + 1.0f;
    a[i] = x;
  }
}
"""


def _asm(tmp_path, flags):
    from sparse_attention_kv_hisparse_amd.build import HIPCC
    src = tmp_path / "k.hip"
    src.write_text(KERNEL)
    out = tmp_path / "k.s"
    subprocess.check_call([HIPCC, *flags, "--cuda-device-only", "-S", str(src), "-o", str(out)],
                          stderr=subprocess.DEVNULL)
    return out.read_text()


def test_device_code_has_no_packed_fp32(tmp_path):
    from sparse_attention_kv_hisparse_amd.build import FLAGS, HIPCC
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
    with_switch = _asm(tmp_path, flags)
    assert "v_fma_f32" in with_switch or "v_fmac_f32" in with_switch
    assert "v_pk_fma_f32" not in with_switch and "v_pk_mul_f32" not in with_switch \
        and "v_pk_add_f32" not in with_switch
    i = flags.index("-packed-fp32-ops")
    control = _asm(tmp_path, flags[:i - 3] + flags[i + 1:])
    assert "v_pk_fma_f32" in control

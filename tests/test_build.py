"""CPU: the device code is built without packed fp32 VALU instructions.

The library is compiled with the packed-fp32-ops target feature turned off;
this test compiles each HIP source to gfx950 assembly with the build's own
flags and checks that no v_pk_add_f32 / v_pk_mul_f32 / v_pk_fma_f32 appears.
"""

import os
import re
import subprocess

import pytest

from gemm_lora_shrink_amd import build as B


@pytest.mark.parametrize("src", B.SOURCES)
def test_no_packed_fp32_in_device_code(src, tmp_path):
    out = tmp_path / (src + ".s")
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-fPIC", "-fvisibility=hidden")]
    cmd = [B.hipcc(), *flags, "-I", os.path.join(B.ROOT, "include"), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    asm = out.read_text()
    bad = re.findall(r"\bv_pk_(?:add|mul|fma)_f32\b", asm)
    assert not bad, f"{src}: {len(bad)} packed fp32 instructions"

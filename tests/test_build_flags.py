"""The HIP kernels must contain no packed-fp32 instructions (v_pk_add_f32,
v_pk_mul_f32, v_pk_fma_f32): the build disables them and this checks the
device assembly the build's own flags produce (CPU only, needs hipcc)."""
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("kvc_build", os.path.join(ROOT, "paged_kv_cache_split_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="no hipcc")
def test_no_packed_fp32_in_device_code(tmp_path):
    b = _build_module()
    flags = [f for f in b.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / "kernels.s"
    cmd = [b.hipcc(), *flags, "-S", "--offload-device-only", os.path.join(b.CSRC, "kvc_kernels.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    asm = out.read_text()
    assert "v_mfma_f32_16x16x32_bf16" in asm          # sanity: this is the decode code
    bad = re.findall(r"v_pk_(?:add|mul|fma)_f32", asm)
    assert not bad, f"{len(bad)} packed-fp32 instructions in device code"

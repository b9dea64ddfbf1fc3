"""Resource use of the compiled kernels (CPU only: hipcc cross-compiles for gfx950).

Every kernel of the library and of the benchmark's probes must run without
private (scratch) memory -- a spill or a dynamically indexed local array lands
there and turns a streaming pass into a latency-bound one -- and within 128
VGPRs, so that at least four waves fit on each SIMD.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _kernel_resources(src, tmp_path):
    from optimizer_step_tensor_amd import build as B
    out = str(tmp_path / (os.path.basename(src) + ".s"))
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", "-o", out, src], check=True,
                   stderr=subprocess.DEVNULL)
    text = open(out).read()
    res = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S):
        body = m.group(2)
        scratch = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body).group(1))
        vgpr = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", body).group(1))
        res[m.group(1)] = (scratch, vgpr)
    return res


@pytest.mark.parametrize("name", ["kernels.hip", "ceiling.hip"])
def test_no_scratch_and_bounded_vgprs(name, tmp_path):
    src = os.path.join(ROOT, "optimizer_step_tensor_amd", "csrc", name)
    res = _kernel_resources(src, tmp_path)
    assert len(res) >= (20 if name == "kernels.hip" else 4), sorted(res)
    scratch = {k: v for k, v in res.items() if v[0] != 0}
    assert scratch == {}, scratch
    wide = {k: v for k, v in res.items() if v[1] > 128}
    assert wide == {}, wide

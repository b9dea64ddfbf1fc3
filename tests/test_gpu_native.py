"""The C ABI without PyTorch (needs a GPU): optimizer_step_tensor_amd/examples/c_api_step,
a plain HIP program built by __graft_entry__.build(), runs three updates on hipMalloc'd buffers
(the second with token weights computed on the device and both micro-batches folded in as one
group, the third with the weights computed inside the first accumulation) and checks them
against closed forms (exact sum of squares, the token weights, the first three AdamW steps)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXAMPLE = os.path.join(ROOT, "optimizer_step_tensor_amd", "examples", "c_api_step")


def test_c_example_runs_a_step():
    assert os.path.exists(EXAMPLE), "the C example is not built; run __graft_entry__.build()"
    r = subprocess.run([EXAMPLE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and " ok " in r.stdout

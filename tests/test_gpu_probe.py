"""The matrix-core probe used to report the reachable MFMA rate beside the spec."""
import pytest
import torch

import variable_length_sequence_amd as vl
from gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs_and_rate_is_plausible():
    dev = require_gpu()
    say("mfma probe 1024 iters x 2048 workgroups")
    sink = torch.full((2048,), float("nan"), dtype=torch.float32, device=dev)
    vl.varlen_mfma_probe(64, 2048, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flops = vl.varlen_mfma_probe(1024, 2048, sink)
    e1.record()
    torch.cuda.synchronize()
    assert flops == 2048 * 4 * 1024 * 8 * 2 * 32 * 32 * 16
    assert torch.isfinite(sink).all()
    tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    say(f"probe {tflops:.0f} TFLOP/s")
    assert 200 < tflops < 2600       # below the 2516.6 TFLOP/s spec, far above a broken launch


def test_mfma_probe_rejects_bad_arguments():
    require_gpu()
    with pytest.raises(vl.VarlenError):
        vl.varlen_mfma_probe(0, 16)

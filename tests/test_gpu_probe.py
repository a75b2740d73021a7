"""The MFMA throughput probe that the benchmark reads its sustained-peak
figure from: it runs, keeps its products live, and reports a rate below the
published bf16 peak."""

import pytest
import torch

import bench
from long_context_exact_blockwise_amd import ringattn as ra
from tests._gpu_common import cuda

pytestmark = pytest.mark.gpu


def test_probe_mfma_rate_is_plausible():
    wgs = 256
    out = torch.full((wgs * ra.PROBE_THREADS,), float("nan"), dtype=torch.float32, device=cuda())
    ra.ringattn_probe_mfma(out, wgs, 10)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    rate = bench.probe_peak(cuda(), iters=20000, reps=1)
    print(f"probed bf16 MFMA rate {rate:.1f} TFLOP/s")
    assert 0.3 * bench.PEAK_BF16_TFLOPS < rate <= 1.02 * bench.PEAK_BF16_TFLOPS

"""The MFMA throughput probes that the benchmark reads its sustained-peak
figures from: they run, keep their products live, and report rates below the
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


def test_probe_mfma_with_random_operands():
    wgs = 256
    out = torch.full((wgs * ra.PROBE_THREADS,), float("nan"), dtype=torch.float32, device=cuda())
    g = torch.Generator(device=cuda())
    g.manual_seed(0)
    ops = torch.randn(wgs * ra.PROBE_THREADS * ra.PROBE_OPERANDS_PER_THREAD, generator=g, device=cuda()).to(
        torch.bfloat16)
    ra.ringattn_probe_mfma_data(ops, out, wgs, 10)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    # ten products of N(0, 1) bf16 fragments: the accumulators are far from zero
    assert out.abs().max() > 1.0
    rate = bench.probe_peak(cuda(), iters=20000, reps=1, random_operands=True)
    print(f"probed bf16 MFMA rate, random operands {rate:.1f} TFLOP/s")
    assert 0.3 * bench.PEAK_BF16_TFLOPS < rate <= 1.02 * bench.PEAK_BF16_TFLOPS


@pytest.mark.parametrize("lds_reads", [16, 4])
def test_probe_mfma_with_operands_from_lds(lds_reads):
    wgs = 256
    out = torch.full((wgs * ra.PROBE_THREADS,), float("nan"), dtype=torch.float32, device=cuda())
    g = torch.Generator(device=cuda())
    g.manual_seed(1)
    ops = torch.randn(wgs * ra.PROBE_THREADS * ra.PROBE_OPERANDS_PER_THREAD, generator=g, device=cuda()).to(
        torch.bfloat16)
    ra.ringattn_probe_mfma_lds(ops, out, wgs, 3, lds_reads)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert out.abs().max() > 1.0  # 48 products of N(0, 1) bf16 fragments
    rate = bench.probe_peak(cuda(), iters=20000, reps=1, lds_reads=lds_reads)
    print(f"probed bf16 MFMA rate, random operands, {lds_reads} LDS reads per 16 products: {rate:.1f} TFLOP/s")
    assert 0.3 * bench.PEAK_BF16_TFLOPS < rate <= 1.02 * bench.PEAK_BF16_TFLOPS

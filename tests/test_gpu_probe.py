"""The matrix-core rate probe (a measurement aid of bench.py): it runs through
the C ABI, reports the FLOP count of its launch, and writes finite sums."""
import pytest
import torch

import associative_memory_amd as am

pytestmark = pytest.mark.gpu


def test_probe_runs_and_counts():
    sink = torch.full((8 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flops = am.kata_probe_mfma_bf16(sink, 8, 100)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 100 * 8 * 2 * 16 * 16 * 32
    assert bool(torch.isfinite(sink).all()) and float(sink.min()) > 0.0

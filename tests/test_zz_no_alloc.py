"""kata_forward_chunked_noalloc through the C ABI: the entry point that keeps
its workspace in the library's static device scratch instead of caller
memory.  Two calls in a row (the second on a smaller input, so the scratch
still holds the first call's larger state) must each reproduce
kata_forward_chunked's output bits and meet the parity bar against the fp64
oracle.  (Its validation paths, including shapes beyond the scratch limit,
are host tests of the ABI.)"""
import numpy as np
import pytest
import torch

import associative_memory_amd as am
import kata_inputs as ki
from oracle import kata_oracle as orc
from gpu_util import check, say, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _case(B, H, T, d, chunk, seed):
    inp = ki.forward_inputs(B, H, T, d, 64, ki.BF16, seed=seed)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    return inp, q, k, v


@pytest.mark.parametrize("scan", ["sequential", "associative", "fused"])
def test_noalloc_matches_workspace_entry_point(scan):
    cases = [(4, 8, 2048, 16, 64, 1), (1, 2, 1000, 16, 128, 2), (1, 3, 3000, 32, 64, 3)]
    outs = []
    for (B, H, T, d, chunk, seed) in cases:
        need = am.kata_forward_workspace_bytes(B, H, T, d, 64, chunk, scan)
        say(f"noalloc B{B} H{H} T{T} d{d} C{chunk} scan={scan}: workspace {need} bytes")
        assert 0 < need <= am.KATA_NOALLOC_SCRATCH_BYTES
        inp, q, k, v = _case(B, H, T, d, chunk, seed)
        out = torch.empty((B, H, T, 64), dtype=torch.bfloat16, device="cuda")
        am.kata_forward_chunked_noalloc(q, k, v, chunk, scan=scan, out=out)
        ref_dev = am.kata_forward_chunked(q, k, v, chunk, scan=scan)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_dev.view(torch.int16)), "bits differ"
        ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6)
        check(to_host64(out), ref, ki.BF16, np.abs(inp.v64).max(), f"noalloc {(B, H, T, d, chunk)}")
        outs.append(out)
    # the first output is untouched by the later calls
    assert outs[0].shape == (4, 8, 2048, 64)

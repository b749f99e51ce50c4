"""GPU parity of the quadratic (O(T^2)) forward against the fp64 oracle,
through the C ABI: full outputs at the T = 2048 workload and on ragged shapes,
sampled rows at T = 8192 (d = 32), the KATA-Mg block maps at d = 64 (full
outputs on ragged shapes, sampled rows at the page's Table 8 shape),
agreement with the chunked form, and run-to-run determinism."""
import numpy as np
import pytest
import torch

import associative_memory_amd as am
import kata_inputs as ki
from oracle import kata_oracle as orc
from gpu_util import assert_guards, check, guarded, say, to_dev, to_host64

pytestmark = pytest.mark.gpu


def run(inp, eps, g=1):
    q, k, v = (to_dev(a, inp.dtype) for a in (inp.q, inp.k, inp.v))
    out = am.kata_forward_quadratic(q, k, v, eps=eps, g=g)
    torch.cuda.synchronize()
    return to_host64(out)


def test_full_parity_medium():
    w = ki.MEDIUM
    say(f"quadratic {w.name}")
    inp = ki.workload_inputs(w)
    got = run(inp, w.eps)
    ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, w.eps)
    check(got, ref, w.dtype, np.abs(inp.v64).max(), "quadratic " + w.name)


QUAD_CASES = [
    # (B, H, T, d)
    (1, 1, 1, 16), (1, 2, 77, 16), (1, 1, 129, 16), (2, 3, 1000, 16), (1, 2, 4097, 16),
    (3, 1, 128, 32), (2, 2, 300, 32), (1, 1, 5000, 32), (1, 1, 8191, 16),
]


@pytest.mark.parametrize("case", QUAD_CASES, ids=lambda c: "B{}H{}T{}d{}".format(*c))
def test_ragged_and_edge_shapes(case):
    B, H, T, d = case
    say(f"quadratic ragged {case}")
    inp = ki.forward_inputs(B, H, T, d, 64, ki.BF16, seed=T + 3 * d)
    got = run(inp, 1e-6)
    ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6)
    check(got, ref, ki.BF16, np.abs(inp.v64).max(), f"quadratic {case}")


def test_sampled_rows_wide():
    w = ki.WIDE
    say(f"quadratic {w.name} sampled rows")
    inp = ki.workload_inputs(w)
    got = run(inp, w.eps)
    g = np.random.Generator(np.random.PCG64(w.seed + 200))
    refs, gots = [], []
    for b in range(w.B):
        for h in range(w.H):
            rows = sorted({0, 1, 127, 128, w.T - 1} | {int(x) for x in g.integers(0, w.T, 12)})
            refs.append(orc.forward_rows(inp.q64[b, h], inp.k64[b, h], inp.v64[b, h], rows, w.eps))
            gots.append(got[b, h, rows])
    check(np.concatenate(gots), np.concatenate(refs), w.dtype, np.abs(inp.v64).max(), "quadratic wide rows")


BLOCK_CASES = [
    # (B, H, T, d, g): block width d/g in {16, 32, 64}
    (1, 1, 1, 64, 1), (1, 2, 77, 64, 2), (2, 1, 300, 64, 4), (1, 1, 1000, 64, 1),
    (1, 2, 2049, 64, 2), (2, 2, 513, 64, 4), (1, 1, 4097, 64, 4), (2, 1, 700, 32, 2),
    (1, 1, 3000, 32, 2), (2, 4, 1024, 64, 2),
]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=lambda c: "B{}H{}T{}d{}g{}".format(*c))
def test_block_maps(case):
    B, H, T, d, g = case
    say(f"quadratic block map {case}")
    inp = ki.forward_inputs(B, H, T, d, 64, ki.BF16, seed=T + 7 * g)
    got = run(inp, 1e-6, g)
    ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6, g=g)
    check(got, ref, ki.BF16, np.abs(inp.v64).max(), f"quadratic {case}")


@pytest.mark.parametrize("g", [1, 2, 4])
def test_table8_shape_sampled_rows(g):
    w = ki.table8(4096, g, 40 + g)
    say(f"quadratic {w.name} sampled rows")
    inp = ki.workload_inputs(w)
    got = run(inp, w.eps, g)
    rng = np.random.Generator(np.random.PCG64(w.seed + 300))
    refs, gots = [], []
    for b in range(w.B):
        for h in rng.choice(w.H, 4, replace=False):
            rows = sorted({0, 127, 128, w.T - 1} | {int(x) for x in rng.integers(0, w.T, 6)})
            refs.append(orc.forward_rows(inp.q64[b, h], inp.k64[b, h], inp.v64[b, h], rows, w.eps, g=g))
            gots.append(got[b, h, rows])
    check(np.concatenate(gots), np.concatenate(refs), w.dtype, np.abs(inp.v64).max(), w.name + " rows")


def test_matches_chunked_form():
    # the two forms compute the same read; both are bf16-rounded at the end
    B, H, T, d = 2, 2, 3000, 16
    inp = ki.forward_inputs(B, H, T, d, 64, ki.BF16, seed=31)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    a = to_host64(am.kata_forward_quadratic(q, k, v))
    b = to_host64(am.kata_forward_chunked(q, k, v, 128))
    torch.cuda.synchronize()
    assert np.abs(a - b).max() <= 2e-2 * np.abs(inp.v64).max()


def test_deterministic():
    inp = ki.forward_inputs(1, 3, 2500, 32, 64, ki.BF16, seed=8)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    x = am.kata_forward_quadratic(q, k, v)
    y = am.kata_forward_quadratic(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("d,g", [(16, 1), (32, 1), (64, 1), (64, 2), (64, 4)])
def test_guard_bands(d, g):
    B, H, T = 2, 3, 333
    say(f"quadratic guard bands d={d} g={g}")
    inp = ki.forward_inputs(B, H, T, d, 64, ki.BF16, seed=d + g)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    buf, out = guarded((B, H, T, 64), torch.bfloat16)
    am.kata_forward_quadratic(q, k, v, g=g, out=out)
    torch.cuda.synchronize()
    assert_guards(buf, f"quadratic d={d} g={g}")
    ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6, g=g)
    check(to_host64(out), ref, ki.BF16, np.abs(inp.v64).max(), f"guarded quadratic d={d} g={g}")

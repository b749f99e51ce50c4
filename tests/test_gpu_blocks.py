"""GPU parity of the chunked read at d = 64 with the KATA-Mg maps against the
fp64 oracle, through the C ABI: KATA-M4 (four blocks of 16), KATA-M2 (two
blocks of 32, two slices of the feature axis) and the full map KATA-M1 (four
slices).  Full outputs on ragged and multi-span shapes, sampled rows at the
page's Table 8 shape (B = 8, H = 16, d_head = 64) up to the T = 131072 the
benchmark times, at T = 65536,
agreement with the quadratic form of the same map, both prefix variants, and
determinism."""
import numpy as np
import pytest
import torch

import associative_memory_amd as am
import kata_inputs as ki
from oracle import kata_oracle as orc
from gpu_util import (assert_guards, assert_workspace_guard, check, guarded, guarded_workspace, say,
                      to_dev, to_host64)

pytestmark = pytest.mark.gpu

GS = [4, 2, 1]


def run(inp, g, eps=1e-6, scan="auto"):
    q, k, v = (to_dev(a, inp.dtype) for a in (inp.q, inp.k, inp.v))
    out = am.kata_forward_chunked_blocks(q, k, v, g, eps=eps, scan=scan)
    torch.cuda.synchronize()
    return to_host64(out)


CASES = [
    # (B, H, T): one token, partial / exact / ragged chunks, several chunks,
    # multi-span plans
    (1, 1, 1), (1, 2, 63), (1, 1, 64), (2, 1, 65), (1, 2, 1000), (2, 2, 4097), (1, 1, 20000),
    (1, 3, 33333),
]


@pytest.mark.parametrize("g", GS)
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}T{}".format(*c))
def test_ragged_and_multispan(case, g):
    B, H, T = case
    say(f"chunked M{g} {case}")
    inp = ki.forward_inputs(B, H, T, 64, 64, ki.BF16, seed=T + 11 + g)
    got = run(inp, g)
    ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6, g=g)
    check(got, ref, ki.BF16, np.abs(inp.v64).max(), f"chunked M{g} {case}")


@pytest.mark.parametrize("g", GS)
@pytest.mark.parametrize("scan", ["sequential", "associative"])
def test_table8_shape_sampled_rows(scan, g):
    w = ki.table8(4096, g, 45)
    say(f"chunked {w.name} sampled rows, {scan} prefix")
    inp = ki.workload_inputs(w)
    got = run(inp, g, w.eps, scan)
    rng = np.random.Generator(np.random.PCG64(46))
    refs, gots = [], []
    for b in range(w.B):
        for h in rng.choice(w.H, 3, replace=False):
            rows = sorted({0, 63, 64, w.T - 1} | {int(x) for x in rng.integers(0, w.T, 6)})
            refs.append(orc.forward_rows(inp.q64[b, h], inp.k64[b, h], inp.v64[b, h], rows, w.eps, g=g))
            gots.append(got[b, h, rows])
    check(np.concatenate(gots), np.concatenate(refs), w.dtype, np.abs(inp.v64).max(), w.name + " rows")


@pytest.mark.parametrize("g", GS)
def test_long_sequence_sampled_rows(g):
    B, H, T = 1, 4, 65536
    say(f"chunked M{g} B{B} H{H} T{T} sampled rows")
    inp = ki.forward_inputs(B, H, T, 64, 64, ki.BF16, seed=47)
    got = run(inp, g)
    rng = np.random.Generator(np.random.PCG64(48))
    refs, gots = [], []
    for h in range(H):
        rows = sorted({0, 64, 4095, T - 1} | {int(x) for x in rng.integers(0, T, 8)})
        refs.append(orc.forward_rows(inp.q64[0, h], inp.k64[0, h], inp.v64[0, h], rows, 1e-6, g=g))
        gots.append(got[0, h, rows])
    check(np.concatenate(gots), np.concatenate(refs), ki.BF16, np.abs(inp.v64).max(), f"chunked M{g} long rows")


@pytest.mark.parametrize("g", GS)
def test_matches_quadratic_form(g):
    inp = ki.forward_inputs(2, 3, 3000, 64, 64, ki.BF16, seed=49)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    a = to_host64(am.kata_forward_chunked_blocks(q, k, v, g))
    b = to_host64(am.kata_forward_quadratic(q, k, v, g=g))
    torch.cuda.synchronize()
    assert np.abs(a - b).max() <= 2e-2 * np.abs(inp.v64).max()


@pytest.mark.parametrize("g", GS)
def test_deterministic(g):
    inp = ki.forward_inputs(1, 2, 9000, 64, 64, ki.BF16, seed=50)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    x = am.kata_forward_chunked_blocks(q, k, v, g)
    y = am.kata_forward_chunked_blocks(q, k, v, g)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("g", GS)
def test_timed_shape_sampled_rows(g):
    # B = 8, H = 16, T = 131072: the shape and launch plan the benchmark
    # times, inputs drawn on the device as there; sampled rows of 6 heads
    w = ki.table8(131072, g, 70)
    say(f"chunked {w.name} (timed shape) sampled rows")
    q, k, v = ki.forward_inputs_torch(w.B, w.H, w.T, w.d, w.dv, w.seed, "cuda")
    out = am.kata_forward_chunked_blocks(q, k, v, g, chunk=64, eps=w.eps)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(71))
    vmax = float(v.float().abs().max())
    refs, gots = [], []
    for n in range(6):
        b, h = int(rng.integers(0, w.B)), int(rng.integers(0, w.H))
        rows = sorted({0, 64, w.T // 2, w.T - 1} | {int(x) for x in rng.integers(0, w.T, 4)})
        qh, kh, vh = (to_host64(x[b, h]) for x in (q, k, v))
        refs.append(orc.forward_rows(qh, kh, vh, rows, w.eps, g=g))
        gots.append(to_host64(out[b, h, rows]))
    check(np.concatenate(gots), np.concatenate(refs), ki.BF16, vmax, f"{w.name} rows")


@pytest.mark.parametrize("g", GS)
@pytest.mark.parametrize("case", [(1, 2, 1000), (2, 1, 20000)], ids=lambda c: "B{}H{}T{}".format(*c))
def test_guard_bands(case, g):
    B, H, T = case
    say(f"chunked M{g} guard bands {case}")
    inp = ki.forward_inputs(B, H, T, 64, 64, ki.BF16, seed=T + 3 * g)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    buf, out = guarded((B, H, T, 64), torch.bfloat16)
    need = int(am.lib().kata_forward_chunked_blocks_workspace_bytes(B, H, T, 64, 64, g, 64, 0))
    wbuf, ws = guarded_workspace(need)
    am.kata_forward_chunked_blocks(q, k, v, g, out=out, workspace=ws if need else None)
    torch.cuda.synchronize()
    assert_guards(buf, f"M{g} out")
    assert_workspace_guard(wbuf, need, f"M{g} workspace")
    if T <= 1000:
        ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6, g=g)
        check(to_host64(out), ref, ki.BF16, np.abs(inp.v64).max(), f"guarded M{g}")

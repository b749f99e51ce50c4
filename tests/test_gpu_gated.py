"""GPU parity of the gated read (GatedKATA, d = 16 and d = 32, dv = 64)
against the fp64 oracle, through the C ABI: full outputs on ragged and
multi-span shapes at both chunk lengths, gates without decay (the
unnormalised KATA numerator) and with strong decay, sampled rows at
T = 131072 (d = 16) and every row of two heads at T = 8192 (d = 32), guard
bands, and determinism.

Tolerance.  The gated read has no denominator, so |o_t| grows with the
decayed score mass A_t = sum_{s<=t} (prod gamma) (q_t.k_s)^2.  The bf16
roundings (scores, state copy, query features) each cost about 2^-9 of the
terms they touch, so row t is held to 2e-2 max|v| max(1, A_t) -- the
normalised read's bar, 2e-2 max|v|, carried over to the unnormalised sum --
plus the RMS bound of the other parity tests."""
import numpy as np
import pytest
import torch

import associative_memory_amd as am
import kata_inputs as ki
from oracle import kata_oracle as orc
from gpu_util import (RMS_TOL, assert_guards, assert_workspace_guard, guarded, guarded_workspace, say,
                      to_dev, to_host64)

pytestmark = pytest.mark.gpu


def run(inp, lg, chunk):
    q, k, v = (to_dev(a, inp.dtype) for a in (inp.q, inp.k, inp.v))
    g = torch.from_numpy(np.ascontiguousarray(lg, dtype=np.float32)).cuda()
    out = am.kata_forward_gated(q, k, v, g, chunk=chunk)
    torch.cuda.synchronize()
    return to_host64(out)


def check_gated(got, ref, mass, vmax, what):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref).max(axis=-1)
    bar = 2e-2 * vmax * np.maximum(1.0, mass)
    rms_rel = float(np.sqrt(np.mean((got - ref) ** 2)) / np.sqrt(np.mean(ref * ref)))
    worst = float((err / bar).max())
    say(f"  {what}: max err/bar {worst:.3e}, rms_rel {rms_rel:.3e}")
    assert (err <= bar).all(), f"{what}: error above the bar (worst ratio {worst})"
    assert rms_rel <= RMS_TOL[ki.BF16], f"{what}: rms rel err {rms_rel}"


def full_check(inp, lg, chunk, what):
    got = run(inp, lg, chunk)
    ref = orc.forward_gated_quadratic(inp.q64, inp.k64, inp.v64, lg.astype(np.float64))
    ones = np.ones(inp.v64.shape[:-1] + (1,))
    mass = orc.forward_gated_quadratic(inp.q64, inp.k64, ones, lg.astype(np.float64))[..., 0]
    check_gated(got, ref, mass, np.abs(inp.v64).max(), what)


GATED_CASES = [
    # (B, H, T, chunk): one token, partial / exact / ragged chunks, several
    # chunks, and multi-span plans
    (1, 1, 1, 128), (1, 2, 100, 64), (1, 1, 128, 128), (2, 1, 129, 128), (1, 2, 1000, 64),
    (2, 2, 4097, 128), (1, 1, 20000, 128), (1, 3, 33333, 64), (1, 1, 9000, 64),
]


@pytest.mark.parametrize("d", [16, 32])
@pytest.mark.parametrize("case", GATED_CASES, ids=lambda c: "B{}H{}T{}C{}".format(*c))
def test_ragged_and_multispan(case, d):
    B, H, T, C = case
    say(f"gated d={d} {case}")
    inp = ki.forward_inputs(B, H, T, d, 64, ki.BF16, seed=T + C + d)
    lg = ki.draw_log_gamma(B, H, T, seed=T + C)
    full_check(inp, lg, C, f"gated d={d} {case}")


@pytest.mark.parametrize("d", [16, 32])
@pytest.mark.parametrize("C", [64, 128])
def test_no_decay_is_the_numerator(C, d):
    # gamma = 1: o_t = sum_{s<=t} (q_t.k_s)^2 v_s, the unnormalised KATA read
    B, H, T = 1, 2, 3000
    inp = ki.forward_inputs(B, H, T, d, 64, ki.BF16, seed=90 + d)
    lg = np.zeros((B, H, T), dtype=np.float32)
    full_check(inp, lg, C, f"gated d={d} no decay C{C}")


@pytest.mark.parametrize("d", [16, 32])
@pytest.mark.parametrize("C", [64, 128])
def test_strong_decay(C, d):
    # gates around 0.5: a memory of a few tokens, far below one chunk
    B, H, T = 2, 2, 2500
    inp = ki.forward_inputs(B, H, T, d, 64, ki.BF16, seed=91 + d)
    rng = np.random.Generator(np.random.PCG64(92))
    lg = (-np.log1p(np.exp(-rng.standard_normal((B, H, T))))).astype(np.float32)
    full_check(inp, lg, C, f"gated d={d} strong decay C{C}")


@pytest.mark.parametrize("C", [64, 128])
def test_d32_workload_shape_two_heads(C):
    # B = 2, H = 16, T = 8192, d = 32 (the d = 32 forward workload's shape and
    # plan): every row of the first and last head
    w = ki.WIDE
    say(f"gated {w.name} C{C}: every row of two heads")
    inp = ki.workload_inputs(w)
    lg = ki.draw_log_gamma(w.B, w.H, w.T, seed=w.seed)
    got = run(inp, lg, C)
    vmax = np.abs(inp.v64).max()
    for (b, h) in ((0, 0), (w.B - 1, w.H - 1)):
        q, k, v, g = inp.q64[b, h], inp.k64[b, h], inp.v64[b, h], lg[b, h].astype(np.float64)
        ref = orc.forward_gated_quadratic(q, k, v, g)
        mass = orc.forward_gated_quadratic(q, k, np.ones((w.T, 1)), g)[..., 0]
        check_gated(got[b, h], ref, mass, vmax, f"gated {w.name} C{C} head ({b},{h})")


def test_long_sequence_sampled_rows():
    w = ki.LONG
    say(f"gated {w.name} sampled rows")
    inp = ki.workload_inputs(w)
    lg = ki.draw_log_gamma(w.B, w.H, w.T, seed=w.seed)
    got = run(inp, lg, w.chunk)
    rng = np.random.Generator(np.random.PCG64(93))
    refs, gots, masses = [], [], []
    for h in rng.choice(w.H, 4, replace=False):
        rows = sorted({0, 127, 128, 4095, w.T - 1} | {int(x) for x in rng.integers(0, w.T, 8)})
        q, k, v, g = inp.q64[0, h], inp.k64[0, h], inp.v64[0, h], lg[0, h].astype(np.float64)
        refs.append(orc.forward_gated_rows(q, k, v, g, rows))
        masses.append(orc.forward_gated_rows(q, k, np.ones((w.T, 1)), g, rows)[:, 0])
        gots.append(got[0, h, rows])
    check_gated(np.concatenate(gots), np.concatenate(refs), np.concatenate(masses),
                np.abs(inp.v64).max(), "gated long rows")


def test_many_spans_sampled_rows():
    # one head of 40000 tokens at chunk 64: 313 spans, so the affine prefix
    # is the reduce-then-scan form with two passes over each segment
    B, H, T, C = 1, 1, 40000, 64
    say(f"gated B{B} H{H} T{T} C{C} sampled rows")
    inp = ki.forward_inputs(B, H, T, 16, 64, ki.BF16, seed=95)
    lg = ki.draw_log_gamma(B, H, T, seed=95)
    got = run(inp, lg, C)
    rng = np.random.Generator(np.random.PCG64(96))
    rows = sorted({0, 63, 64, 127, 128, T // 2, T - 1} | {int(x) for x in rng.integers(0, T, 16)})
    q, k, v, g = inp.q64[0, 0], inp.k64[0, 0], inp.v64[0, 0], lg[0, 0].astype(np.float64)
    ref = orc.forward_gated_rows(q, k, v, g, rows)
    mass = orc.forward_gated_rows(q, k, np.ones((T, 1)), g, rows)[:, 0]
    check_gated(got[0, 0, rows], ref, mass, np.abs(inp.v64).max(), "gated many spans")


@pytest.mark.parametrize("d", [16, 32])
def test_deterministic(d):
    inp = ki.forward_inputs(1, 4, 7000, d, 64, ki.BF16, seed=94)
    lg = torch.from_numpy(ki.draw_log_gamma(1, 4, 7000, seed=94)).cuda()
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    x = am.kata_forward_gated(q, k, v, lg)
    y = am.kata_forward_gated(q, k, v, lg)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("d", [16, 32])
@pytest.mark.parametrize("C", [64, 128])
@pytest.mark.parametrize("case", [(1, 2, 1000), (2, 1, 20000)], ids=lambda c: "B{}H{}T{}".format(*c))
def test_guard_bands(case, C, d):
    B, H, T = case
    say(f"gated d={d} guard bands {case} C{C}")
    inp = ki.forward_inputs(B, H, T, d, 64, ki.BF16, seed=T + C + 1)
    lg = ki.draw_log_gamma(B, H, T, seed=T + C + 1)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    buf, out = guarded((B, H, T, 64), torch.bfloat16)
    need = am.kata_forward_gated_workspace_bytes(B, H, T, d, 64, C)
    wbuf, ws = guarded_workspace(need)
    am.kata_forward_gated(q, k, v, torch.from_numpy(lg).cuda(), chunk=C, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert_guards(buf, "gated out")
    assert_workspace_guard(wbuf, need, "gated workspace")
    if T <= 1000:
        ref = orc.forward_gated_quadratic(inp.q64, inp.k64, inp.v64, lg.astype(np.float64))
        mass = orc.forward_gated_quadratic(inp.q64, inp.k64, np.ones((B, H, T, 1)), lg.astype(np.float64))[..., 0]
        check_gated(to_host64(out), ref, mass, np.abs(inp.v64).max(), "guarded gated")

"""GPU parity of the chunked forward against the fp64 oracle, through the C ABI.

Every workload is compared element by element over every output: the small
ones against the plain definition, the long ones (T = 8192 at d = 32,
T = 131072) in the launch configuration the benchmark times against the fp64
chunked form (itself pinned to the definition) and on sampled rows of every
head against the definition.  Guard bands around the output and past the
workspace catch writes outside them on every kernel family.
"""
import functools

import numpy as np
import pytest
import torch

import associative_memory_amd as am
import kata_inputs as ki
from oracle import kata_oracle as orc
from gpu_util import (assert_guards, assert_workspace_guard, check, guarded, guarded_workspace, say,
                      to_dev, to_host64)

pytestmark = pytest.mark.gpu

SCANS = ("sequential", "associative")


def run(inp: ki.ForwardInputs, chunk, eps, scan="auto"):
    q, k, v = (to_dev(a, inp.dtype) for a in (inp.q, inp.k, inp.v))
    out = am.kata_forward_chunked(q, k, v, chunk, eps=eps, scan=scan)
    torch.cuda.synchronize()
    return to_host64(out)


@pytest.mark.parametrize("scan", SCANS)
@pytest.mark.parametrize("w", [ki.TINY, ki.MEDIUM], ids=lambda w: w.name)
def test_full_parity_small_workloads(w, scan):
    say(f"forward {w.name} scan={scan}")
    inp = ki.workload_inputs(w)
    got = run(inp, w.chunk, w.eps, scan)
    ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, w.eps)
    check(got, ref, w.dtype, np.abs(inp.v64).max(), w.name)


def _sampled_rows(T, chunk, g, n=24):
    rows = {0, 1, chunk - 1, chunk, chunk + 1, T // 2, T - 2, T - 1}
    rows.update(int(x) for x in g.integers(0, T, n))
    return sorted(r for r in rows if 0 <= r < T)


@functools.lru_cache(maxsize=2)
def _long_case(w):
    """Inputs of a long workload and the fp64 chunked oracle over every head
    (Eqs. 17-20, pinned to the plain definition by the oracle's own tests;
    under a second per head of host time at these sizes)."""
    inp = ki.workload_inputs(w)
    ref = orc.forward_chunked(inp.q64, inp.k64, inp.v64, w.chunk, w.eps)
    return inp, ref


@pytest.mark.parametrize("scan", SCANS)
@pytest.mark.parametrize("w", [ki.WIDE, ki.LONG], ids=lambda w: w.name)
def test_full_parity_long_workloads(w, scan):
    # every output of every head, in the launch configuration the benchmark
    # times, against the chunked oracle; sampled rows of every head against
    # the plain definition as well
    say(f"forward {w.name} scan={scan} plan: "
        + am.kata_forward_plan(w.B, w.H, w.T, w.d, w.dv, w.chunk, am.KATA_BF16, scan))
    inp, ref = _long_case(w)
    got = run(inp, w.chunk, w.eps, scan)
    vmax = np.abs(inp.v64).max()
    check(got, ref, w.dtype, vmax, f"{w.name} every output")
    g = np.random.Generator(np.random.PCG64(w.seed + 100))
    refs, gots = [], []
    for b in range(w.B):
        for h in range(w.H):
            rows = _sampled_rows(w.T, w.chunk, g, n=8)
            refs.append(orc.forward_rows(inp.q64[b, h], inp.k64[b, h], inp.v64[b, h], rows, w.eps))
            gots.append(got[b, h, rows])
    check(np.concatenate(gots), np.concatenate(refs), w.dtype, vmax, f"{w.name} sampled rows (definition)")


def _plan_fields(plan):
    return {k: v for k, v in (f.split("=", 1) for f in plan.split())}


@pytest.mark.parametrize("scan", SCANS)
@pytest.mark.parametrize("shape", [(4, 8, 16384, 64), (4, 8, 32768, 128)], ids=lambda s: "B{}H{}T{}C{}".format(*s))
def test_paired_spans_boundaries(shape, scan):
    # plans with paired spans (even spans G + G/8 chunks, odd spans the rest
    # of 2G): the first and last rows of every span of sampled heads, plus
    # random rows of every head
    B, H, T, chunk = shape
    plan = am.kata_forward_plan(B, H, T, 16, 64, chunk, am.KATA_BF16, scan)
    say(f"forward paired spans {shape} scan={scan} plan: {plan}")
    f = _plan_fields(plan)
    G, GL, n_spans = int(f["chunks_per_span"]), int(f["paired_even_span"]), int(f["n_spans"])
    assert GL > G, "the plan does not pair spans"
    starts = [((j // 2) * 2 * G + (GL if j % 2 else 0)) * chunk for j in range(n_spans + 1)]
    assert starts[-1] == T
    inp = ki.forward_inputs(B, H, T, 16, 64, ki.BF16, seed=T + chunk)
    got = run(inp, chunk, 1e-6, scan)
    g = np.random.Generator(np.random.PCG64(T + 1))
    edges = sorted({r for s in starts[1:-1] for r in (s - 1, s)} | {0, T - 1})
    refs, gots = [], []
    for b in range(B):
        for h in range(H):
            rows = sorted(set(int(x) for x in g.integers(0, T, 6)) | (set(edges) if (b + h) % 3 == 0 else set()))
            refs.append(orc.forward_rows(inp.q64[b, h], inp.k64[b, h], inp.v64[b, h], rows, 1e-6))
            gots.append(got[b, h, rows])
    check(np.concatenate(gots), np.concatenate(refs), ki.BF16, np.abs(inp.v64).max(), f"paired spans {shape}")


@pytest.mark.parametrize("T", [1 << 22, (1 << 22) + 333], ids=["T4194304", "T4194637"])
def test_sequences_far_beyond_the_benchmark(T):
    # two heads of 4M tokens (32x the benchmarked length): 64-bit offsets, a
    # 256-span plan (paired spans when the chunks divide evenly, a ragged last
    # span otherwise) and the associative prefix the library picks there.
    # Inputs are drawn on the device (the host draw would take minutes);
    # each head is copied back for the oracle rows.
    B, H, d, dv, chunk = 1, 2, 16, 64, 128
    plan = am.kata_forward_plan(B, H, T, d, dv, chunk, am.KATA_BF16, "auto")
    say(f"forward B{B} H{H} T{T} plan: {plan}")
    assert "scan=associative" in plan
    q, k, v = ki.forward_inputs_torch(B, H, T, d, dv, seed=T % 1000, device="cuda")
    out = am.kata_forward_chunked(q, k, v, chunk, eps=1e-6)
    torch.cuda.synchronize()
    g = np.random.Generator(np.random.PCG64(T))
    vmax = float(v.float().abs().max())
    refs, gots = [], []
    for h in range(H):
        rows = sorted({0, chunk - 1, chunk, T // 2, T - 1} | {int(x) for x in g.integers(0, T, 8)})
        qh, kh, vh = (to_host64(x[0, h]) for x in (q, k, v))
        refs.append(orc.forward_rows(qh, kh, vh, rows, 1e-6))
        gots.append(to_host64(out[0, h, rows]))
        del qh, kh, vh
    check(np.concatenate(gots), np.concatenate(refs), ki.BF16, vmax, f"T{T} rows")


def test_many_spans_sampled_rows():
    # one head of 70001 tokens at chunk 64: 365 spans of 3 chunks, so the
    # associative prefix reduces segments of 23 spans in two passes
    B, H, T, d, dv, chunk = 1, 1, 70001, 16, 64, 64
    plan = am.kata_forward_plan(B, H, T, d, dv, chunk, am.KATA_BF16, "auto")
    say(f"forward B{B} H{H} T{T} plan: {plan}")
    assert "scan=associative" in plan and "n_spans=365" in plan
    inp = ki.forward_inputs(B, H, T, d, dv, ki.BF16, seed=97)
    got = run(inp, chunk, 1e-6)
    rng = np.random.Generator(np.random.PCG64(98))
    rows = sorted({0, 191, 192, T // 2, T - 1} | {int(x) for x in rng.integers(0, T, 16)})
    ref = orc.forward_rows(inp.q64[0, 0], inp.k64[0, 0], inp.v64[0, 0], rows, 1e-6)
    check(got[0, 0, rows], ref, ki.BF16, np.abs(inp.v64).max(), "many spans")


RAGGED = [
    # (B, H, T, d, dv, chunk, dtype)
    (1, 1, 1, 16, 16, 32, ki.F32),
    (1, 2, 77, 16, 64, 128, ki.BF16),
    (2, 3, 1000, 16, 64, 64, ki.BF16),
    (3, 2, 1000, 32, 32, 128, ki.BF16),
    (2, 1, 333, 32, 16, 32, ki.F32),
    (1, 3, 4099, 16, 32, 64, ki.F32),
    (1, 1, 5000, 32, 64, 64, ki.BF16),
    (1, 1, 129, 16, 64, 128, ki.BF16),
    (3, 5, 2500, 16, 64, 128, ki.BF16),
    (2, 2, 8191, 16, 64, 64, ki.BF16),
    (1, 3, 40000, 16, 64, 128, ki.BF16),
    (2, 3, 3000, 32, 64, 128, ki.BF16),
    (1, 2, 9000, 32, 64, 64, ki.BF16),
    (3, 1, 65, 32, 64, 64, ki.BF16),
]


@pytest.mark.parametrize("scan", SCANS)
@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "B{}H{}T{}d{}dv{}C{}{}".format(*c))
def test_ragged_and_edge_shapes(case, scan):
    B, H, T, d, dv, chunk, dtype = case
    say(f"forward ragged {case} scan={scan}")
    inp = ki.forward_inputs(B, H, T, d, dv, dtype, seed=T + d + dv)
    got = run(inp, chunk, 1e-6, scan)
    ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6)
    check(got, ref, dtype, np.abs(inp.v64).max(), str(case))


def test_deterministic_run_to_run():
    w = ki.MEDIUM
    inp = ki.workload_inputs(w)
    q, k, v = (to_dev(a, inp.dtype) for a in (inp.q, inp.k, inp.v))
    for scan in SCANS:
        a = am.kata_forward_chunked(q, k, v, w.chunk, eps=w.eps, scan=scan)
        b = am.kata_forward_chunked(q, k, v, w.chunk, eps=w.eps, scan=scan)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_chunk_size_invariance_and_guard_bands():
    B, H, T, d, dv = 2, 2, 1500, 16, 64
    inp = ki.forward_inputs(B, H, T, d, dv, ki.F32, seed=77)
    q, k, v = (to_dev(a, ki.F32) for a in (inp.q, inp.k, inp.v))
    outs = []
    for chunk in (32, 64, 128):
        # out inside a larger buffer with canaries on both sides
        pad = 1024
        buf = torch.full((pad + B * H * T * dv + pad,), 12345.0, device="cuda")
        out = buf[pad:pad + B * H * T * dv].view(B, H, T, dv)
        am.kata_forward_chunked(q, k, v, chunk, eps=1e-6, out=out)
        torch.cuda.synchronize()
        assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[-pad:] == 12345.0)
        outs.append(to_host64(out))
    ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6)
    for o in outs:
        check(o, ref, ki.F32, np.abs(inp.v64).max(), "chunk invariance")
    assert np.abs(outs[0] - outs[2]).max() <= 2e-4 * np.abs(inp.v64).max()


def test_symmetries_on_device():
    # sign flips of q/k rows and a common rotation leave the read unchanged
    B, H, T, d, dv = 1, 2, 700, 16, 32
    inp = ki.forward_inputs(B, H, T, d, dv, ki.F32, seed=5)
    g = np.random.Generator(np.random.PCG64(6))
    U, _ = np.linalg.qr(g.standard_normal((d, d)))
    sgn = g.choice([-1.0, 1.0], size=(B, H, T, 1))
    q2 = (inp.q64 * sgn) @ U.T
    k2 = (inp.k64 * sgn[..., ::-1, :]) @ U.T
    base = run(inp, 64, 1e-6)
    alt = ki.ForwardInputs(q2.astype(np.float32), k2.astype(np.float32), inp.v, q2, k2, inp.v64, ki.F32)
    rot = run(alt, 64, 1e-6)
    ref = orc.forward_quadratic(q2.astype(np.float32).astype(np.float64),
                                k2.astype(np.float32).astype(np.float64), inp.v64, 1e-6)
    check(rot, ref, ki.F32, np.abs(inp.v64).max(), "rotated")
    assert np.abs(rot - base).max() <= 2e-4 * np.abs(inp.v64).max()


def test_constant_values_reproduced():
    # constant v: o_t = c D_t / (D_t + eps); with unit q, k and T >= 64 the
    # factor is 1 to ~1e-6, an O(1) output the long-T bar can see.
    B, H, T, d, dv = 1, 1, 4096, 16, 64
    inp = ki.forward_inputs(B, H, T, d, dv, ki.BF16, seed=12)
    v = np.zeros_like(inp.v64) + np.linspace(-2, 2, dv)
    vb, v64 = ki.as_storage(v, ki.BF16)
    alt = ki.ForwardInputs(inp.q, inp.k, vb, inp.q64, inp.k64, v64, ki.BF16)
    got = run(alt, 128, 1e-6)
    ref = orc.forward_quadratic(inp.q64, inp.k64, v64, 1e-6)
    check(got, ref, ki.BF16, np.abs(v64).max(), "constant v")
    # beyond the first few tokens the read equals v to bf16 rounding
    assert np.abs(got[0, 0, 64:] - v64[0, 0, 64:]).max() <= 2 ** -7 * 2


@pytest.mark.parametrize("scan", SCANS)
def test_profiled_entry_matches_plain(scan):
    # the benchmark's entry point: same output bits as kata_forward_chunked,
    # and every stage event recorded in order on the library's stream
    import bench

    hip = bench.Hip()
    w = ki.MEDIUM
    inp = ki.workload_inputs(w)
    q, k, v = (to_dev(a, inp.dtype) for a in (inp.q, inp.k, inp.v))
    plain = am.kata_forward_chunked(q, k, v, w.chunk, eps=w.eps, scan=scan)
    ev = am.StageEvents()
    hs = [hip.event() for _ in range(6)]
    for i in range(3):
        ev.stage_begin[i] = hs[2 * i]
        ev.stage_end[i] = hs[2 * i + 1]
    prof = am.kata_forward_chunked_profiled(q, k, v, w.chunk, ev, eps=w.eps, scan=scan)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), prof.view(torch.int16))
    for i in range(3):
        assert hip.ms(hs[2 * i], hs[2 * i + 1]) >= 0.0
    assert hip.ms(hs[1], hs[2]) >= 0.0 and hip.ms(hs[3], hs[4]) >= 0.0  # stages in order
    for h in hs:
        hip.destroy(h)


@pytest.mark.parametrize("chunk", (64, 128))
def test_denominator_edges(chunk):
    # Zero keys over whole spans leave the carried key Gram matrix exactly 0,
    # so those rows read 0 / (0 + eps) = 0; a zero gap in the middle keeps it
    # constant across spans; zero query rows read 0; keys and queries scaled
    # by 4 raise q^T Z q by 256; a large eps weighs in on every row.
    B, H, T, d, dv = 1, 2, 20000, 16, 64
    inp = ki.forward_inputs(B, H, T, d, dv, ki.BF16, seed=91)
    q, k = inp.q64.copy(), inp.k64.copy()
    k[0, 0, :9000] = 0.0
    k[0, 1, 5000:15000] = 0.0
    q[:, :, ::97] = 0.0
    for scale, eps in ((1.0, 1e-6), (4.0, 1e-6), (1.0, 10.0)):
        qs, q64 = ki.as_storage(q * scale, ki.BF16)
        ks, k64 = ki.as_storage(k * scale, ki.BF16)
        alt = ki.ForwardInputs(qs, ks, inp.v, q64, k64, inp.v64, ki.BF16)
        what = f"chunk={chunk} scale={scale} eps={eps}"
        say(f"forward denominator edges {what}")
        got = run(alt, chunk, eps)
        ref = orc.forward_quadratic(q64, k64, inp.v64, eps)
        check(got, ref, ki.BF16, np.abs(inp.v64).max(), what)
        assert np.all(got[0, 0, :9000] == 0.0), "rows with no nonzero key before them"
        assert np.all(got[:, :, ::97] == 0.0), "zero query rows"


GUARD_CASES = [
    # (B, H, T, d, chunk): the d = 16 DMA readout with a ragged last chunk and
    # a ragged span, paired spans, a single span; the d = 32 kernels ragged
    (1, 2, 77, 16, 128),
    (2, 3, 1000, 16, 64),
    (4, 8, 16384, 16, 64),
    (1, 1, 5000, 16, 128),
    (3, 2, 1000, 32, 128),
    (1, 2, 9000, 32, 64),
    (1, 1, 65, 32, 64),
]


@pytest.mark.parametrize("scan", SCANS)
@pytest.mark.parametrize("case", GUARD_CASES, ids=lambda c: "B{}H{}T{}d{}C{}".format(*c))
def test_guard_bands_bf16(case, scan):
    B, H, T, d, chunk = case
    dv = 64
    say(f"forward guard bands {case} scan={scan}")
    inp = ki.forward_inputs(B, H, T, d, dv, ki.BF16, seed=T + 5 * d)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    buf, out = guarded((B, H, T, dv), torch.bfloat16)
    need = am.kata_forward_workspace_bytes(B, H, T, d, dv, chunk, scan)
    wbuf, ws = guarded_workspace(need)
    am.kata_forward_chunked(q, k, v, chunk, eps=1e-6, scan=scan, out=out, workspace=ws if need else None)
    torch.cuda.synchronize()
    assert_guards(buf, f"out {case}")
    assert_workspace_guard(wbuf, need, f"workspace {case}")
    ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6) if T <= 9000 else None
    if ref is not None:
        check(to_host64(out), ref, ki.BF16, np.abs(inp.v64).max(), f"guarded {case}")


RECOMPUTE_CASES = [
    # (B, H, T, chunk), d = 16, dv = 64, bf16: the T = 2048 workload at both
    # chunk sizes, a single ragged chunk, ragged spans and last chunks, heads
    # of many spans (the latest workgroup sums 60 spans before its own)
    (4, 8, 2048, 64),
    (4, 8, 2048, 128),
    (1, 2, 77, 128),
    (2, 3, 1000, 64),
    (1, 1, 5000, 128),
    (3, 5, 2500, 128),
    (2, 2, 8191, 64),
    (1, 3, 40000, 128),
    (1, 1, 1, 64),        # one token, one span
    (7, 9, 65, 64),       # 63 heads of two chunks, the second a single token
    (40, 16, 300, 64),    # more heads than workgroups: one span per head
]


@pytest.mark.parametrize("case", RECOMPUTE_CASES, ids=lambda c: "B{}H{}T{}C{}".format(*c))
def test_recompute_prefix(case):
    """Prefix formed inside the readout workgroups (no span sums, no prefix
    launch, no workspace): every output against the oracle, guard bands
    around the output, and run-to-run bitwise determinism."""
    B, H, T, chunk = case
    d, dv = 16, 64
    plan = am.kata_forward_plan(B, H, T, d, dv, chunk, am.KATA_BF16, "recompute")
    say(f"forward recompute {case} plan: {plan}")
    assert "scan=recompute" in plan and "wg_state=0" in plan and "workspace_bytes=0" in plan
    assert am.kata_forward_workspace_bytes(B, H, T, d, dv, chunk, "recompute") == 0
    inp = ki.forward_inputs(B, H, T, d, dv, ki.BF16, seed=T + 11 * chunk)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    buf, out = guarded((B, H, T, dv), torch.bfloat16)
    am.kata_forward_chunked(q, k, v, chunk, eps=1e-6, scan="recompute", out=out)
    again = am.kata_forward_chunked(q, k, v, chunk, eps=1e-6, scan="recompute")
    torch.cuda.synchronize()
    assert_guards(buf, f"out {case}")
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "run-to-run bits"
    if T <= 9000:
        ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6)
    else:
        ref = orc.forward_chunked(inp.q64, inp.k64, inp.v64, chunk, 1e-6)
    check(to_host64(out), ref, ki.BF16, np.abs(inp.v64).max(), f"recompute {case}")


FUSED_CASES = [
    # (B, H, T, chunk), d = 16, dv = 64, bf16: the T = 2048 workload at both
    # chunk sizes (the automatic plan there), ragged spans and last chunks,
    # head counts that are not a multiple of the 8 XCDs, many spans per head
    # (the latest workgroup adds 63 span sums), one token, one span per head
    (4, 8, 2048, 64),
    (4, 8, 2048, 128),
    (2, 3, 1000, 64),
    (3, 5, 2500, 128),
    (1, 1, 5000, 128),
    (2, 2, 8191, 64),
    (1, 3, 40000, 128),
    (1, 1, 1, 64),
    (7, 9, 65, 64),
    (40, 16, 300, 64),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "B{}H{}T{}C{}".format(*c))
def test_fused_prefix(case):
    """Prefix added in the readout from the stored span sums: every output
    against the oracle, guard bands around the output, run-to-run bitwise
    determinism, and the same bits as the sequential prefix whenever the two
    plans cut the same spans (the sums are added in the same order)."""
    B, H, T, chunk = case
    d, dv = 16, 64
    plan = am.kata_forward_plan(B, H, T, d, dv, chunk, am.KATA_BF16, "fused")
    seq_plan = am.kata_forward_plan(B, H, T, d, dv, chunk, am.KATA_BF16, "sequential")
    say(f"forward fused {case} plan: {plan}")
    assert "scan=fused" in plan and "paired_even_span=0" in plan
    inp = ki.forward_inputs(B, H, T, d, dv, ki.BF16, seed=T + 13 * chunk)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    buf, out = guarded((B, H, T, dv), torch.bfloat16)
    am.kata_forward_chunked(q, k, v, chunk, eps=1e-6, scan="fused", out=out)
    again = am.kata_forward_chunked(q, k, v, chunk, eps=1e-6, scan="fused")
    seq = am.kata_forward_chunked(q, k, v, chunk, eps=1e-6, scan="sequential")
    torch.cuda.synchronize()
    assert_guards(buf, f"out {case}")
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "run-to-run bits"
    if plan.replace("scan=fused", "") == seq_plan.replace("scan=sequential", ""):
        assert torch.equal(out.view(torch.int16), seq.view(torch.int16)), "fused vs sequential bits"
    if T <= 9000:
        ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6)
    else:
        ref = orc.forward_chunked(inp.q64, inp.k64, inp.v64, chunk, 1e-6)
    check(to_host64(out), ref, ki.BF16, np.abs(inp.v64).max(), f"fused {case}")


FUSED_CAPPED_CASES = [
    # (B, H, T, chunk), d = 16: few heads at short T, where the automatic
    # plan takes 16 spans of at most 256 tokens with the fused prefix; a
    # ragged last span and last chunk
    (2, 8, 2048, 64),
    (1, 8, 4096, 64),
    (1, 1, 2048, 64),
    (1, 3, 3001, 64),
]


@pytest.mark.parametrize("case", FUSED_CAPPED_CASES, ids=lambda c: "B{}H{}T{}C{}".format(*c))
def test_fused_prefix_capped_spans(case):
    """The automatic plan's 16 short spans with the fused prefix: every output
    against the oracle, guard bands and run-to-run bitwise determinism."""
    B, H, T, chunk = case
    d, dv = 16, 64
    plan = am.kata_forward_plan(B, H, T, d, dv, chunk, am.KATA_BF16, "auto")
    say(f"forward auto {case} plan: {plan}")
    assert "scan=fused" in plan and "n_spans=16 " in plan
    inp = ki.forward_inputs(B, H, T, d, dv, ki.BF16, seed=T + 7 * chunk)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    buf, out = guarded((B, H, T, dv), torch.bfloat16)
    am.kata_forward_chunked(q, k, v, chunk, eps=1e-6, scan="auto", out=out)
    again = am.kata_forward_chunked(q, k, v, chunk, eps=1e-6, scan="auto")
    torch.cuda.synchronize()
    assert_guards(buf, f"out {case}")
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "run-to-run bits"
    ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6)
    check(to_host64(out), ref, ki.BF16, np.abs(inp.v64).max(), f"fused capped {case}")


FUSED32_CASES = [
    # (B, H, T), d = 32, dv = 64, chunk 64, bf16: 2 and 4 spans per head (the
    # automatic plan there), the d = 32 workload's 8 spans, ragged spans and a
    # head count that is not a multiple of 8
    (8, 16, 2048),
    (4, 16, 2048),
    (2, 16, 8192),
    (3, 5, 2500),
    (1, 1, 1),
]


@pytest.mark.parametrize("case", FUSED32_CASES, ids=lambda c: "B{}H{}T{}".format(*c))
def test_fused_prefix_d32(case):
    """The wave-specialised d = 32 readout with the prefix added from the
    stored span sums: the sequential prefix's bits (same spans, same order),
    guard bands, and sampled rows of every head against the oracle."""
    B, H, T = case
    d, dv, chunk = 32, 64, 64
    plan = am.kata_forward_plan(B, H, T, d, dv, chunk, am.KATA_BF16, "fused")
    say(f"forward fused d=32 {case} plan: {plan}")
    assert "scan=fused" in plan
    q, k, v = ki.forward_inputs_torch(B, H, T, d, dv, seed=T + 5, device="cuda")
    buf, out = guarded((B, H, T, dv), torch.bfloat16)
    am.kata_forward_chunked(q, k, v, chunk, eps=1e-6, scan="fused", out=out)
    seq = am.kata_forward_chunked(q, k, v, chunk, eps=1e-6, scan="sequential")
    torch.cuda.synchronize()
    assert_guards(buf, f"out {case}")
    assert torch.equal(out.view(torch.int16), seq.view(torch.int16)), "fused vs sequential bits"
    g = np.random.Generator(np.random.PCG64(T))
    vmax = float(v.float().abs().max())
    refs, gots = [], []
    for b in range(B):
        for h in range(H):
            rows = sorted({0, T - 1} | {int(x) for x in g.integers(0, T, 3)})
            qh, kh, vh = (to_host64(x[b, h]) for x in (q, k, v))
            refs.append(orc.forward_rows(qh, kh, vh, rows, 1e-6))
            gots.append(to_host64(out[b, h, rows]))
    check(np.concatenate(gots), np.concatenate(refs), ki.BF16, vmax, f"fused d=32 {case} rows")


def _random_cases(n=36, seed=2026):
    """Seeded shapes across every plan the forward can take: both head
    widths, both chunk lengths, every prefix mode, lengths from one token to
    a few thousand (ragged last chunks and spans), head counts that are and
    are not multiples of the 8 XCDs."""
    g = np.random.Generator(np.random.PCG64(seed))
    scans = ["auto", "sequential", "associative", "recompute", "fused"]
    out = []
    while len(out) < n:
        d = int(g.choice([16, 32]))
        chunk = int(g.choice([64, 128]))
        scan = str(g.choice(scans))
        if scan == "recompute" and d != 16:
            continue
        if scan == "fused" and d == 32 and chunk == 128:
            continue
        B, H = int(g.integers(1, 4)), int(g.integers(1, 9))
        T = int(g.choice([1, 2, 63, 64, 65, 127, 129, 500, 1000, 2047, 2048, 2049, 3000, 4100]))
        out.append((B, H, T, d, chunk, scan))
    return out


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: "B{}H{}T{}d{}C{}-{}".format(*c))
def test_random_shapes_every_plan(case):
    """Every output against the definition, guard bands around the output
    and past the workspace, on seeded shapes across the plans."""
    B, H, T, d, chunk, scan = case
    dv = 64
    plan = am.kata_forward_plan(B, H, T, d, dv, chunk, am.KATA_BF16, scan)
    say(f"forward random {case} plan: {plan}")
    inp = ki.forward_inputs(B, H, T, d, dv, ki.BF16, seed=7 * T + B + 3 * H + d + chunk)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    need = am.kata_forward_workspace_bytes(B, H, T, d, dv, chunk, scan)
    wbuf, ws = guarded_workspace(need)
    buf, out = guarded((B, H, T, dv), torch.bfloat16)
    am.kata_forward_chunked(q, k, v, chunk, eps=1e-6, scan=scan, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert_guards(buf, f"out {case}")
    assert_workspace_guard(wbuf, need, f"workspace {case}")
    ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6)
    check(to_host64(out), ref, ki.BF16, np.abs(inp.v64).max(), f"random {case}")

"""GPU parity of the linear-feature chunked forward against the fp64 oracle,
through the C ABI: the cone maps KATA-Orthant and KATA-Lorentz (normalised
read) and the identity map psi(x) = x (first-order read, no denominator),
D = d = 64, at every chunk length (32, 64, 128) and with both prefixes: full
outputs on ragged and multi-span shapes and at the B = 4, H = 12 shape of the
page's orthant/Lorentz throughput table (App. E.1, chunk 32), sampled rows at
the B = 1, H = 16, T = 131072 shape of its Table 11 (identity map, chunk 128,
and the cone maps), the orthant map without a shift, guard bands and
run-to-run determinism.

Identity-map tolerance.  With signed scores and no denominator |o_t| grows
like the score norm sqrt(A_t), A_t = sum_{s<=t} (q_t.k_s)^2 (about t/64 for
unit rows at d = 64), and the bf16 roundings (scores, the state copy, the
output) each cost about 2^-9 of what they touch, so row t is held to
2e-2 max|v| max(1, sqrt(A_t)) -- the normalised read's bar carried over to
the unnormalised sum, A_t from the oracle -- plus the RMS bound of the other
parity tests."""
import numpy as np
import pytest
import torch

import associative_memory_amd as am
import kata_inputs as ki
from oracle import kata_oracle as orc
from gpu_util import (RMS_TOL, assert_guards, assert_workspace_guard, check, guarded, guarded_workspace,
                      say, to_dev, to_host64)

pytestmark = pytest.mark.gpu

FEATURES = ["orthant", "lorentz"]
ALL_FEATURES = ["orthant", "lorentz", "identity"]
CHUNKS = [32, 64, 128]
SCANS = ["sequential", "associative"]


def run(inp, feature, eps=1e-6, shift=1e-6, chunk=64, scan="auto"):
    q, k, v = (to_dev(a, inp.dtype) for a in (inp.q, inp.k, inp.v))
    out = am.kata_forward_linear(q, k, v, feature=feature, shift=shift, eps=eps, chunk=chunk, scan=scan)
    torch.cuda.synchronize()
    return to_host64(out)


def score_norm(q64, k64):
    """sqrt(sum_{s<=t} (q_t.k_s)^2) per row: the gated oracle with no decay and v = 1."""
    lead = q64.shape[:-1]
    A = orc.forward_gated_quadratic(q64, k64, np.ones(lead + (1,)), np.zeros(lead))[..., 0]
    return np.sqrt(A)


def check_identity(got, ref, norm, vmax, what):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref).max(axis=-1)
    bar = 2e-2 * vmax * np.maximum(1.0, norm)
    rms_rel = float(np.sqrt(np.mean((got - ref) ** 2)) / np.sqrt(np.mean(ref * ref)))
    worst = float((err / bar).max())
    say(f"  {what}: max err/bar {worst:.3e}, rms_rel {rms_rel:.3e}")
    assert (err <= bar).all(), f"{what}: error above the bar (worst ratio {worst})"
    assert rms_rel <= RMS_TOL[ki.BF16], f"{what}: rms rel err {rms_rel}"


def full_check(inp, feature, chunk, scan="auto", what="", eps=1e-6, shift=1e-6):
    got = run(inp, feature, eps, shift, chunk, scan)
    vmax = np.abs(inp.v64).max()
    if feature == "identity":
        ref = orc.forward_identity_quadratic(inp.q64, inp.k64, inp.v64)
        check_identity(got, ref, score_norm(inp.q64, inp.k64), vmax, what)
    else:
        ref = orc.forward_linear_quadratic(inp.q64, inp.k64, inp.v64, feature, eps, shift=shift)
        check(got, ref, ki.BF16, vmax, what)


LIN_CASES = [
    # (B, H, T): one token, a partial chunk, one chunk, a ragged second chunk,
    # several chunks, and multi-span plans (BH * spans ~ 512)
    (1, 1, 1), (1, 2, 63), (1, 1, 64), (2, 1, 65), (1, 2, 1000), (2, 2, 4097), (1, 1, 20000),
]


@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("feature", ALL_FEATURES)
@pytest.mark.parametrize("case", LIN_CASES, ids=lambda c: "B{}H{}T{}".format(*c))
def test_ragged_and_multispan(case, feature, chunk):
    B, H, T = case
    say(f"linear {feature} C{chunk} {case}")
    inp = ki.forward_inputs(B, H, T, 64, 64, ki.BF16, seed=T + (7 if feature == "lorentz" else 0) + chunk)
    full_check(inp, feature, chunk, what=f"linear {feature} C{chunk} {case}")


@pytest.mark.parametrize("scan", SCANS)
@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("feature", ALL_FEATURES)
def test_both_prefixes_many_spans(feature, chunk, scan):
    # one head of 20011 tokens: 313 spans of 2 chunks at chunk 32, 313 of 1
    # at chunk 64, 157 of 1 at chunk 128 (ragged last chunk)
    B, H, T = 1, 1, 20011
    say(f"linear {feature} C{chunk} scan={scan} B{B} H{H} T{T}")
    inp = ki.forward_inputs(B, H, T, 64, 64, ki.BF16, seed=T + chunk)
    full_check(inp, feature, chunk, scan, what=f"linear {feature} C{chunk} {scan} T{T}")


@pytest.mark.parametrize("scan", SCANS)
@pytest.mark.parametrize("feature", FEATURES)
def test_page_table_shape_full(feature, scan):
    # B = 4, H = 12, T = 1024, d = dv = 64 at chunk 32: the shape of the
    # page's orthant/Lorentz throughput table (App. E.1)
    w = ki.ForwardWorkload(f"B4_H12_T1024_d64_dv64_{feature}_C32_bf16", 4, 12, 1024, 64, 64, 32, ki.BF16, 50)
    say(f"linear {w.name} scan={scan}")
    inp = ki.workload_inputs(w)
    full_check(inp, feature, w.chunk, scan, what=f"{w.name} {scan}")


@pytest.mark.parametrize("scan", SCANS)
@pytest.mark.parametrize("feature", ALL_FEATURES)
def test_long_sequence_sampled_rows(feature, scan):
    # B = 1, H = 16, T = 131072 (the page's Table 11 shape) at chunk 128: 32
    # spans of 32 chunks per head; inputs drawn on the device
    B, H, T, C = 1, 16, 131072, 128
    say(f"linear {feature} B{B} H{H} T{T} C{C} scan={scan} sampled rows")
    q, k, v = ki.forward_inputs_torch(B, H, T, 64, 64, 60 + len(feature), "cuda")
    out = am.kata_forward_linear(q, k, v, feature=feature, chunk=C, scan=scan)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(61))
    vmax = float(v.float().abs().max())
    refs, gots, norms = [], [], []
    for h in rng.choice(H, 5, replace=False):
        rows = sorted({0, 127, 128, 4095, 4096, T - 1} | {int(x) for x in rng.integers(0, T, 6)})
        qh, kh, vh = (to_host64(x[0, h]) for x in (q, k, v))
        if feature == "identity":
            refs.append(orc.forward_identity_rows(qh, kh, vh, rows))
            norms.append(np.sqrt(np.array([np.sum((kh[: t + 1] @ qh[t]) ** 2) for t in rows])))
        else:
            refs.append(orc.forward_linear_rows(qh, kh, vh, rows, feature, 1e-6))
        gots.append(to_host64(out[0, h, rows]))
    if feature == "identity":
        check_identity(np.concatenate(gots), np.concatenate(refs), np.concatenate(norms), vmax,
                       f"identity long rows {scan}")
    else:
        check(np.concatenate(gots), np.concatenate(refs), ki.BF16, vmax, f"linear {feature} long rows {scan}")


def test_orthant_without_shift():
    inp = ki.forward_inputs(2, 2, 777, 64, 64, ki.BF16, seed=70)
    got = run(inp, "orthant", eps=1e-6, shift=0.0)
    ref = orc.forward_linear_quadratic(inp.q64, inp.k64, inp.v64, "orthant", 1e-6, shift=0.0)
    check(got, ref, ki.BF16, np.abs(inp.v64).max(), "orthant shift 0")


@pytest.mark.parametrize("feature", ALL_FEATURES)
def test_deterministic(feature):
    inp = ki.forward_inputs(1, 4, 9000, 64, 64, ki.BF16, seed=71)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    for C in CHUNKS:
        x = am.kata_forward_linear(q, k, v, feature=feature, chunk=C)
        y = am.kata_forward_linear(q, k, v, feature=feature, chunk=C)
        torch.cuda.synchronize()
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("feature", ALL_FEATURES)
@pytest.mark.parametrize("case", [(1, 2, 1000), (2, 1, 20000)], ids=lambda c: "B{}H{}T{}".format(*c))
def test_guard_bands(case, feature, chunk):
    B, H, T = case
    say(f"linear {feature} C{chunk} guard bands {case}")
    inp = ki.forward_inputs(B, H, T, 64, 64, ki.BF16, seed=T + 9)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    buf, out = guarded((B, H, T, 64), torch.bfloat16)
    need = am.kata_forward_linear_workspace_bytes(B, H, T, 64, 64, chunk)
    wbuf, ws = guarded_workspace(need)
    am.kata_forward_linear(q, k, v, feature=feature, chunk=chunk, out=out, workspace=ws if need else None)
    torch.cuda.synchronize()
    assert_guards(buf, f"linear {feature} out")
    assert_workspace_guard(wbuf, need, f"linear {feature} workspace")
    if T <= 1000:
        got = to_host64(out)
        vmax = np.abs(inp.v64).max()
        if feature == "identity":
            ref = orc.forward_identity_quadratic(inp.q64, inp.k64, inp.v64)
            check_identity(got, ref, score_norm(inp.q64, inp.k64), vmax, f"guarded identity C{chunk}")
        else:
            ref = orc.forward_linear_quadratic(inp.q64, inp.k64, inp.v64, feature, 1e-6)
            check(got, ref, ki.BF16, vmax, f"guarded linear {feature} C{chunk}")

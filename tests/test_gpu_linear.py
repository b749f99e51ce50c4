"""GPU parity of the linear-feature chunked forward (KATA-Orthant and
KATA-Lorentz, D = d = 64) against the fp64 oracle, through the C ABI: full
outputs on ragged and multi-span shapes and at the B = 4, H = 12 shape of the
page's orthant/Lorentz throughput table (Sec. 4.2), sampled rows at the
B = 1, H = 16, T = 131072 shape of its Table 11, the orthant map without a
shift, and run-to-run determinism."""
import numpy as np
import pytest
import torch

import associative_memory_amd as am
import kata_inputs as ki
from oracle import kata_oracle as orc
from gpu_util import (assert_guards, assert_workspace_guard, check, guarded, guarded_workspace, say,
                      to_dev, to_host64)

pytestmark = pytest.mark.gpu

FEATURES = ["orthant", "lorentz"]


def run(inp, feature, eps=1e-6, shift=1e-6):
    q, k, v = (to_dev(a, inp.dtype) for a in (inp.q, inp.k, inp.v))
    out = am.kata_forward_linear(q, k, v, feature=feature, shift=shift, eps=eps)
    torch.cuda.synchronize()
    return to_host64(out)


LIN_CASES = [
    # (B, H, T): one token, a partial chunk, one chunk, a ragged second chunk,
    # several chunks, and multi-span plans (BH * spans ~ 512)
    (1, 1, 1), (1, 2, 63), (1, 1, 64), (2, 1, 65), (1, 2, 1000), (2, 2, 4097), (1, 1, 20000),
    (1, 3, 33333),
]


@pytest.mark.parametrize("feature", FEATURES)
@pytest.mark.parametrize("case", LIN_CASES, ids=lambda c: "B{}H{}T{}".format(*c))
def test_ragged_and_multispan(case, feature):
    B, H, T = case
    say(f"linear {feature} {case}")
    inp = ki.forward_inputs(B, H, T, 64, 64, ki.BF16, seed=T + (7 if feature == "lorentz" else 0))
    got = run(inp, feature)
    ref = orc.forward_linear_quadratic(inp.q64, inp.k64, inp.v64, feature, 1e-6, shift=1e-6)
    check(got, ref, ki.BF16, np.abs(inp.v64).max(), f"linear {feature} {case}")


@pytest.mark.parametrize("feature", FEATURES)
def test_page_table_shape_full(feature):
    # B = 4, H = 12, T = 1024, d = dv = 64
    w = ki.ForwardWorkload(f"B4_H12_T1024_d64_dv64_{feature}_bf16", 4, 12, 1024, 64, 64, 64, ki.BF16, 50)
    say(f"linear {w.name}")
    inp = ki.workload_inputs(w)
    got = run(inp, feature, w.eps)
    ref = orc.forward_linear_quadratic(inp.q64, inp.k64, inp.v64, feature, w.eps)
    check(got, ref, w.dtype, np.abs(inp.v64).max(), w.name)


@pytest.mark.parametrize("feature", FEATURES)
def test_long_sequence_sampled_rows(feature):
    # B = 1, H = 16, T = 131072: 32 spans of 64 chunks per head
    B, H, T = 1, 16, 131072
    say(f"linear {feature} B{B} H{H} T{T} sampled rows")
    inp = ki.forward_inputs(B, H, T, 64, 64, ki.BF16, seed=60 + len(feature))
    got = run(inp, feature)
    rng = np.random.Generator(np.random.PCG64(61))
    refs, gots = [], []
    for h in rng.choice(H, 6, replace=False):
        rows = sorted({0, 63, 64, 4095, 4096, T - 1} | {int(x) for x in rng.integers(0, T, 8)})
        refs.append(orc.forward_linear_rows(inp.q64[0, h], inp.k64[0, h], inp.v64[0, h], rows, feature, 1e-6))
        gots.append(got[0, h, rows])
    check(np.concatenate(gots), np.concatenate(refs), ki.BF16, np.abs(inp.v64).max(),
          f"linear {feature} long rows")


def test_orthant_without_shift():
    inp = ki.forward_inputs(2, 2, 777, 64, 64, ki.BF16, seed=70)
    got = run(inp, "orthant", eps=1e-6, shift=0.0)
    ref = orc.forward_linear_quadratic(inp.q64, inp.k64, inp.v64, "orthant", 1e-6, shift=0.0)
    check(got, ref, ki.BF16, np.abs(inp.v64).max(), "orthant shift 0")


@pytest.mark.parametrize("feature", FEATURES)
def test_deterministic(feature):
    inp = ki.forward_inputs(1, 4, 9000, 64, 64, ki.BF16, seed=71)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    x = am.kata_forward_linear(q, k, v, feature=feature)
    y = am.kata_forward_linear(q, k, v, feature=feature)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("feature", FEATURES)
@pytest.mark.parametrize("case", [(1, 2, 1000), (2, 1, 20000)], ids=lambda c: "B{}H{}T{}".format(*c))
def test_guard_bands(case, feature):
    B, H, T = case
    say(f"linear {feature} guard bands {case}")
    inp = ki.forward_inputs(B, H, T, 64, 64, ki.BF16, seed=T + 9)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    buf, out = guarded((B, H, T, 64), torch.bfloat16)
    need = am.kata_forward_linear_workspace_bytes(B, H, T, 64, 64, 64)
    wbuf, ws = guarded_workspace(need)
    am.kata_forward_linear(q, k, v, feature=feature, out=out, workspace=ws if need else None)
    torch.cuda.synchronize()
    assert_guards(buf, f"linear {feature} out")
    assert_workspace_guard(wbuf, need, f"linear {feature} workspace")
    if T <= 1000:
        ref = orc.forward_linear_quadratic(inp.q64, inp.k64, inp.v64, feature, 1e-6)
        check(to_host64(out), ref, ki.BF16, np.abs(inp.v64).max(), f"guarded linear {feature}")

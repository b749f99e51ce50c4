"""GPU parity of the feature map, the decode-state prefill and the recurrent
decode step against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import associative_memory_amd as am
import kata_inputs as ki
from oracle import kata_oracle as orc
from gpu_util import assert_guards, check, guarded, say, to_dev, to_host64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [1, 3, 16, 32, 64])
@pytest.mark.parametrize("xd,pd", [(ki.F32, ki.F32), (ki.BF16, ki.F32), (ki.F32, ki.BF16),
                                   (ki.BF16, ki.BF16)])
def test_feature_map(d, xd, pd):
    say(f"feature_map d={d} x={xd} phi={pd}")
    g = np.random.Generator(np.random.PCG64(d))
    rows = 1037
    xs, x64 = ki.as_storage(g.standard_normal((rows, d)), xd)
    x = to_dev(xs, xd)
    phi = am.kata_feature_map(x, phi_dtype=torch.bfloat16 if pd == ki.BF16 else torch.float32)
    torch.cuda.synchronize()
    got = to_host64(phi)
    ref = orc.feature_map(x64)
    # one fp32 product chain then one rounding to the output type
    rel = 2.0 ** -8 if pd == ki.BF16 else 4 * 2.0 ** -24
    assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 1e-30)


def _decode_case(heads, prefill, steps, d, dv, seed, eps=1e-6):
    di = ki.decode_inputs(seed, heads, prefill, steps, d, dv)
    pk = to_dev(di.pk[:, None], ki.F32)  # [heads, 1, P, d] as B = heads, H = 1
    pv = to_dev(di.pv[:, None], ki.F32)
    S, z = am.kata_prefill_state(pk, pv)
    torch.cuda.synchronize()
    S0, z0 = orc.decode_state(di.pk.astype(np.float64), di.pv.astype(np.float64))
    return di, S, z, S0, z0


@pytest.mark.parametrize("d,dv", [(16, 64), (16, 16), (32, 32), (32, 64)])
def test_prefill_state_matches_oracle(d, dv):
    say(f"prefill d={d} dv={dv}")
    di, S, z, S0, z0 = _decode_case(5, 300, 0, d, dv, seed=3)
    Sg, zg = to_host64(S), to_host64(z)
    # fp32 sums of 300 products of magnitude <= max|v|
    bound = 300 * 4 * 2.0 ** -24 * (1 + np.abs(di.pv).max())
    assert np.abs(Sg - S0).max() <= bound
    assert np.abs(zg - z0).max() <= 300 * 4 * 2.0 ** -24


@pytest.mark.parametrize("d,dv,dtype", [(16, 64, ki.F32), (16, 16, ki.F32), (32, 64, ki.F32),
                                        (16, 64, ki.BF16)])
def test_decode_steps_match_oracle(d, dv, dtype):
    say(f"decode d={d} dv={dv} dtype={dtype}")
    heads, prefill, steps, eps = 7, 200, 24, 1e-6
    di, S, z, S_ref, z_ref = _decode_case(heads, prefill, steps, d, dv, seed=11)
    vmax = max(np.abs(di.pv).max(), np.abs(di.sv).max())
    gots, refs = [], []
    for s in range(steps):
        qs, q64 = ki.as_storage(di.sq[s], dtype)
        ks, k64 = ki.as_storage(di.sk[s], dtype)
        vs, v64 = ki.as_storage(di.sv[s], dtype)
        out = am.kata_decode_step(S, z, to_dev(qs, dtype), to_dev(ks, dtype), to_dev(vs, dtype),
                                  eps=eps)
        S_ref, z_ref, o = orc.decode_step(S_ref, z_ref, q64, k64, v64, eps)
        gots.append(to_host64(out))
        refs.append(o)
    torch.cuda.synchronize()
    check(np.stack(gots), np.stack(refs), dtype, vmax, f"decode d={d} dv={dv}")
    np.testing.assert_allclose(to_host64(S), S_ref, rtol=0, atol=1e-4 * vmax)


def test_decode_continues_forward():
    # history through the forward and the prefill, then decode steps, equals
    # the forward over the whole sequence at the new positions
    B, H, T0, n, d, dv = 2, 2, 640, 16, 16, 64
    inp = ki.forward_inputs(B, H, T0 + n, d, dv, ki.F32, seed=21)
    q, k, v = (to_dev(a, ki.F32) for a in (inp.q, inp.k, inp.v))
    full = am.kata_forward_chunked(q, k, v, 64, eps=1e-6)
    S, z = am.kata_prefill_state(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous())
    outs = []
    for t in range(T0, T0 + n):
        o = am.kata_decode_step(S, z, q[:, :, t].reshape(B * H, d).contiguous(),
                                k[:, :, t].reshape(B * H, d).contiguous(),
                                v[:, :, t].reshape(B * H, dv).contiguous(), eps=1e-6)
        outs.append(o.reshape(B, H, dv))
    torch.cuda.synchronize()
    dec = to_host64(torch.stack(outs, dim=2))
    ref = orc.forward_quadratic(inp.q64, inp.k64, inp.v64, 1e-6)[:, :, T0:]
    vmax = np.abs(inp.v64).max()
    check(dec, ref, ki.F32, vmax, "decode after prefill")
    check(to_host64(full)[:, :, T0:], ref, ki.F32, vmax, "forward tail")


def test_checkpoint_resume_bitwise():
    heads, d, dv = 64, 16, 64
    di = ki.decode_inputs(31, heads, 128, 40, d, dv)
    pk = to_dev(di.pk[:, None], ki.F32)
    pv = to_dev(di.pv[:, None], ki.F32)
    S, z = am.kata_prefill_state(pk, pv)
    S2, z2 = S.clone(), z.clone()
    step = lambda S_, z_, s: am.kata_decode_step(S_, z_, to_dev(di.sq[s], ki.F32),
                                                 to_dev(di.sk[s], ki.F32), to_dev(di.sv[s], ki.F32))
    a = [step(S, z, s) for s in range(40)]
    for s in range(20):
        step(S2, z2, s)
    S3, z3 = S2.cpu().to("cuda"), z2.cpu().to("cuda")  # round trip through host memory
    b = [step(S3, z3, s) for s in range(20, 40)]
    torch.cuda.synchronize()
    for x, y in zip(a[20:], b):
        assert torch.equal(x, y)
    assert torch.equal(S, S3) and torch.equal(z, z3)


def test_decode_full_size_all_steps():
    # the 4096-head workload at its configured length: all 1024 steps on the
    # device (every head), every step's output and the final state of eight
    # heads spread over the range against the recurrence in fp64
    w = ki.DECODE
    say(f"decode full size {w.name}: drawing inputs on the device")
    steps = w.steps
    pk, pv, sq, sk, sv = ki.decode_inputs_torch(w.seed, w.heads, w.prefill, steps, w.d, w.dv, "cuda")
    S, z = am.kata_prefill_state(pk[:, None], pv[:, None])
    heads = torch.tensor([0, 1, 17, 1000, 2047, 3333, 4094, 4095], device="cuda")
    outs = torch.empty((steps, len(heads), w.dv), dtype=torch.float32, device="cuda")
    out = torch.empty((w.heads, w.dv), dtype=torch.float32, device="cuda")
    for s in range(steps):
        am.kata_decode_step(S, z, sq[s], sk[s], sv[s], eps=w.eps, out=out)
        outs[s] = out.index_select(0, heads)
    torch.cuda.synchronize()
    say(f"  {steps} steps done; oracle on {len(heads)} heads")
    vmax = max(float(pv.abs().max()), float(sv.abs().max()))
    hs = heads.cpu().tolist()
    S_ref, z_ref = orc.decode_state(pk[hs].double().cpu().numpy(), pv[hs].double().cpu().numpy())
    q64, k64, v64 = (x[:, hs].double().cpu().numpy() for x in (sq, sk, sv))
    refs = []
    for s in range(steps):
        S_ref, z_ref, o = orc.decode_step(S_ref, z_ref, q64[s], k64[s], v64[s], w.eps)
        refs.append(o)
    check(to_host64(outs), np.stack(refs), ki.F32, vmax, f"decode {steps} steps, sampled heads")
    # fp32 sums of prefill + steps terms, each at most 2 max|v| (S) or 2 (z)
    n = w.prefill + steps
    Sg, zg = to_host64(S[heads]), to_host64(z[heads])
    assert np.abs(Sg - S_ref).max() <= n * 4 * 2.0 ** -24 * 2 * (1 + vmax)
    assert np.abs(zg - z_ref).max() <= n * 4 * 2.0 ** -24 * 2


@pytest.mark.parametrize("d,dv", [(16, 64), (32, 16)])
def test_decode_guard_bands(d, dv):
    # S, z and out inside larger buffers: prefill, additive and gated steps
    # write nothing outside them
    heads, prefill, steps = 37, 100, 5
    say(f"decode guard bands d={d} dv={dv}")
    di = ki.decode_inputs(17, heads, prefill, steps, d, dv)
    D = d * (d + 1) // 2
    sbuf, S = guarded((heads, D, dv), torch.float32)
    zbuf, z = guarded((heads, D), torch.float32)
    obuf, out = guarded((heads, dv), torch.float32)
    am.kata_prefill_state(to_dev(di.pk[:, None], ki.F32), to_dev(di.pv[:, None], ki.F32), S=S, z=z)
    S_ref, z_ref = orc.decode_state(di.pk.astype(np.float64), di.pv.astype(np.float64))
    vmax = max(np.abs(di.pv).max(), np.abs(di.sv).max())
    for s in range(steps):
        am.kata_decode_step(S, z, to_dev(di.sq[s], ki.F32), to_dev(di.sk[s], ki.F32),
                            to_dev(di.sv[s], ki.F32), out=out)
        S_ref, z_ref, o = orc.decode_step(S_ref, z_ref, di.sq[s], di.sk[s], di.sv[s], 1e-6)
        torch.cuda.synchronize()
        check(to_host64(out), o, ki.F32, vmax, f"guarded decode step {s}")
    lg = torch.full((heads,), -0.1, dtype=torch.float32, device="cuda")
    am.kata_decode_step_gated(S, to_dev(di.sq[0], ki.F32), to_dev(di.sk[0], ki.F32),
                              to_dev(di.sv[0], ki.F32), lg, out=out)
    torch.cuda.synchronize()
    for buf, what in ((sbuf, "S"), (zbuf, "z"), (obuf, "out")):
        assert_guards(buf, f"decode {what}")


def test_decode_graph_replay_matches_eager():
    # a run of decode steps captured in one HIP graph: every replay (state
    # restored by eager work between replays) equals the eager launches bitwise
    heads, d, dv, n = 96, 16, 64, 12
    say(f"decode graph replay heads={heads} steps={n}")
    di = ki.decode_inputs(41, heads, 64, n, d, dv)
    S0, z0 = am.kata_prefill_state(to_dev(di.pk[:, None], ki.F32), to_dev(di.pv[:, None], ki.F32))
    sq, sk, sv = (to_dev(x, ki.F32) for x in (di.sq, di.sk, di.sv))
    S, z = S0.clone(), z0.clone()
    eager = [am.kata_decode_step(S, z, sq[s], sk[s], sv[s]).clone() for s in range(n)]
    S_e, z_e = S.clone(), z.clone()
    torch.cuda.synchronize()

    S, z = S0.clone(), z0.clone()
    outs = torch.zeros((n, heads, dv), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=cap):
        for s in range(n):
            am.kata_decode_step(S, z, sq[s], sk[s], sv[s], out=outs[s])
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        S.copy_(S0)
        z.copy_(z0)
        outs.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(n):
            assert torch.equal(outs[s], eager[s]), (rep, s)
        assert torch.equal(S, S_e) and torch.equal(z, z_e), rep


@pytest.mark.parametrize("d,dv,dtype", [(16, 64, ki.F32), (16, 16, ki.F32), (32, 64, ki.F32),
                                        (16, 64, ki.BF16)])
def test_gated_decode_steps_match_oracle(d, dv, dtype):
    # GatedKATA steps from the gated state of a history (kata_prefill_state_gated).
    # No denominator: row bars scale with the decayed score mass A =
    # phi(q)^T z_gated, tracked by running the oracle with v = 1.
    say(f"gated decode d={d} dv={dv} dtype={dtype}")
    heads, prefill, steps = 9, 200, 24
    di = ki.decode_inputs(13, heads, prefill, steps, d, dv)
    rng = np.random.Generator(np.random.PCG64(14))
    lg_pre = (-np.log1p(np.exp(-(rng.standard_normal((heads, prefill)) + 3.0)))).astype(np.float32)
    lg = (-np.log1p(np.exp(-(rng.standard_normal((steps, heads)) + 2.0)))).astype(np.float32)
    S = am.kata_prefill_state_gated(to_dev(di.pk[:, None], ki.F32), to_dev(di.pv[:, None], ki.F32),
                                    torch.from_numpy(lg_pre[:, None]).cuda())
    torch.cuda.synchronize()
    pk, pv, lgp = di.pk.astype(np.float64), di.pv.astype(np.float64), lg_pre.astype(np.float64)
    S_ref = np.stack([orc.gated_state(pk[h], pv[h], lgp[h]) for h in range(heads)])
    M_ref = np.stack([orc.gated_state(pk[h], np.ones((prefill, 1)), lgp[h]) for h in range(heads)])
    vmax = max(np.abs(di.pv).max(), np.abs(di.sv).max())
    # the prefilled state itself: fp32, prefill terms each at most 2 max|v|
    assert np.abs(to_host64(S) - S_ref).max() <= prefill * 8 * 2.0 ** -24 * 2 * (1 + vmax)
    tol = 1e-4 if dtype == ki.F32 else 2e-2
    for s in range(steps):
        qs, q64 = ki.as_storage(di.sq[s].astype(np.float64), dtype)
        ks, k64 = ki.as_storage(di.sk[s].astype(np.float64), dtype)
        vs, v64 = ki.as_storage(di.sv[s].astype(np.float64), dtype)
        g = torch.from_numpy(lg[s]).cuda()
        out = am.kata_decode_step_gated(S, to_dev(qs, dtype), to_dev(ks, dtype), to_dev(vs, dtype), g)
        torch.cuda.synchronize()
        S_ref, o_ref = orc.decode_step_gated(S_ref, q64, k64, v64, lg[s].astype(np.float64))
        M_ref, mass = orc.decode_step_gated(M_ref, q64, k64, np.ones((heads, 1)), lg[s].astype(np.float64))
        err = np.abs(to_host64(out) - o_ref).max(axis=-1)
        bar = tol * vmax * np.maximum(1.0, mass[:, 0])
        assert (err <= bar).all(), f"step {s}: worst err/bar {(err / bar).max()}"
    # the state itself, after 24 decays and writes (fp32 throughout)
    Sg = to_host64(S)
    assert np.abs(Sg - S_ref).max() <= 1e-5 * (1 + np.abs(S_ref).max())


@pytest.mark.parametrize("d", [16, 32])
def test_gated_forward_prefill_then_decode(d):
    # a gated history through the forward and the gated prefill, then gated
    # decode steps, equals the gated forward over the whole sequence at the
    # new positions (the unrolled read of Sec. 5.2)
    B, H, T0, n, dv = 2, 2, 700, 12, 64
    say(f"gated forward -> prefill -> decode d={d}")
    inp = ki.forward_inputs(B, H, T0 + n, d, dv, ki.BF16, seed=27 + d)
    lg = ki.draw_log_gamma(B, H, T0 + n, seed=28)
    q, k, v = (to_dev(a, ki.BF16) for a in (inp.q, inp.k, inp.v))
    g = torch.from_numpy(lg).cuda()
    full = am.kata_forward_gated(q, k, v, g)
    S = am.kata_prefill_state_gated(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(),
                                    g[:, :, :T0].contiguous())
    outs = []
    for t in range(T0, T0 + n):
        o = am.kata_decode_step_gated(S, q[:, :, t].reshape(B * H, d).contiguous(),
                                      k[:, :, t].reshape(B * H, d).contiguous(),
                                      v[:, :, t].reshape(B * H, dv).contiguous(),
                                      g[:, :, t].reshape(B * H).contiguous())
        outs.append(o.reshape(B, H, dv))
    torch.cuda.synchronize()
    dec = to_host64(torch.stack(outs, dim=2))
    lg64 = lg.astype(np.float64)
    ref = orc.forward_gated_quadratic(inp.q64, inp.k64, inp.v64, lg64)[:, :, T0:]
    mass = orc.forward_gated_quadratic(inp.q64, inp.k64, np.ones((B, H, T0 + n, 1)), lg64)[:, :, T0:, 0]
    vmax = np.abs(inp.v64).max()
    # bf16 inputs and outputs (fp32 state and arithmetic): the bf16 bar on the mass scale
    err = np.abs(dec - ref).max(axis=-1)
    assert (err <= 2e-2 * vmax * np.maximum(1.0, mass)).all(), f"decode after gated prefill: {err.max()}"
    # the gated prefill itself against the unrolled state (fp32 sums of bf16 products)
    S_ref = np.stack([orc.gated_state(inp.k64[b, h, :T0], inp.v64[b, h, :T0], lg64[b, h, :T0])
                      for b in range(B) for h in range(H)])
    S0 = am.kata_prefill_state_gated(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(),
                                     g[:, :, :T0].contiguous())
    torch.cuda.synchronize()
    assert np.abs(to_host64(S0) - S_ref).max() <= T0 * 8 * 2.0 ** -24 * 2 * (1 + vmax)
    # the forward itself (bf16 path) at the same positions
    errf = np.abs(to_host64(full)[:, :, T0:] - ref).max(axis=-1)
    assert (errf <= 2e-2 * vmax * np.maximum(1.0, mass)).all(), f"gated forward tail: {errf.max()}"

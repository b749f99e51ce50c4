"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/kata.h declares, sizes and plans are consistent, and
every validation error path returns its status without touching the device.
"""
import ctypes
import os
import re

import pytest

import associative_memory_amd as am

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kata.h")

pytestmark = pytest.mark.skipif(not os.path.exists(am.LIB_PATH),
                                reason="libkata.so not built (run __graft_entry__.build())")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
F32, BF16 = 0, 1


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kata_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = am.lib()
    syms = declared_symbols()
    assert len(syms) >= 8
    for s in syms:
        assert hasattr(L, s), f"{s} declared in kata.h but not exported"
    assert sorted(am.EXPORTED) == syms


def test_status_strings_and_feature_dim():
    assert am.status_string(0) == "KATA_OK"
    assert am.status_string(3) == "KATA_ERR_WORKSPACE"
    assert am.status_string(99) == "KATA_ERR_UNKNOWN"
    assert [am.kata_feature_dim(d) for d in (1, 2, 16, 32, 64)] == [1, 3, 136, 528, 2080]
    assert am.kata_feature_dim(0) == -1


def test_workspace_and_plan_consistent():
    L = am.lib()
    for (B, H, T, d, dv, C) in [(1, 1, 256, 16, 16, 32), (4, 8, 2048, 16, 64, 64),
                                (2, 16, 8192, 32, 64, 64), (1, 8, 131072, 16, 64, 128),
                                (1, 1, 1, 16, 16, 32), (3, 2, 1000, 32, 32, 128)]:
        for scan in (0, 1, 2):
            ws = L.kata_forward_workspace_bytes(B, H, T, d, dv, C, scan)
            for dt in (F32, BF16):
                plan = am.kata_forward_plan(B, H, T, d, dv, C, dt, scan)
                fields = dict(kv.split("=") for kv in plan.split())
                assert int(fields["workspace_bytes"]) <= ws
                n_chunks = -(-T // C)
                assert int(fields["n_chunks"]) == n_chunks
                G, n_spans = int(fields["chunks_per_span"]), int(fields["n_spans"])
                assert G * n_spans >= n_chunks > G * (n_spans - 1)
                if scan == 1:
                    assert fields["scan"] == "sequential"
                if scan == 2:
                    assert fields["scan"] == "associative"
    # bf16, d = 16, dv = 64, chunk 64/128 take the matrix-core path
    assert "path=mfma" in am.kata_forward_plan(1, 8, 131072, 16, 64, 128, BF16, 0)
    assert "path=mfma" in am.kata_forward_plan(4, 8, 2048, 16, 64, 64, BF16, 0)
    assert "path=valu" in am.kata_forward_plan(1, 8, 131072, 16, 64, 128, F32, 0)
    assert "path=valu" in am.kata_forward_plan(1, 8, 4096, 16, 64, 32, BF16, 0)
    assert "path=mfma" in am.kata_forward_plan(2, 16, 8192, 32, 64, 64, BF16, 0)
    assert "path=mfma" in am.kata_forward_plan(2, 16, 8192, 32, 64, 128, BF16, 0)
    assert "path=valu" in am.kata_forward_plan(2, 16, 8192, 32, 32, 64, BF16, 0)
    assert L.kata_forward_workspace_bytes(0, 1, 16, 16, 16, 32, 0) == 0
    assert L.kata_forward_workspace_bytes(1, 1, 16, 24, 16, 32, 0) == 0


# Fake, aligned, distinct "device" addresses: validation must reject before
# any use of them.
P = [ctypes.c_void_p((i + 1) << 36) for i in range(8)]
NULL = None


def fwd(q=P[0], k=P[1], v=P[2], out=P[3], B=1, H=1, T=64, d=16, dv=16, C=32, eps=1e-6,
        dt=BF16, scan=0, ws=P[4], wsb=1 << 30, stream=None):
    return am.lib().kata_forward_chunked(q, k, v, out, B, H, T, d, dv, C, eps, dt, scan, ws, wsb,
                                         stream)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), INVALID), (dict(k=NULL), INVALID), (dict(v=NULL), INVALID),
    (dict(out=NULL), INVALID),
    (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(T=0), INVALID),
    (dict(d=24), UNSUPPORTED), (dict(d=64), UNSUPPORTED), (dict(dv=48), UNSUPPORTED),
    (dict(C=16), UNSUPPORTED), (dict(C=256), UNSUPPORTED),
    (dict(eps=-1e-6), INVALID), (dict(eps=float("nan")), INVALID), (dict(eps=float("inf")), INVALID),
    (dict(dt=7), INVALID), (dict(scan=5), INVALID),
    # the prefix formed in the readout (scan 3): bf16, d = 16, dv = 64, chunk 64 / 128 only
    (dict(scan=3), UNSUPPORTED), (dict(scan=3, dv=64, dt=F32), UNSUPPORTED),
    (dict(scan=3, d=32, dv=64, C=64), UNSUPPORTED), (dict(scan=3, dv=64, C=32), UNSUPPORTED),
    # the prefix added in the readout from stored span sums (scan 4): the same shapes
    (dict(scan=4), UNSUPPORTED), (dict(scan=4, dv=64, dt=F32), UNSUPPORTED),
    (dict(scan=4, d=32, dv=64, C=128), UNSUPPORTED), (dict(scan=4, dv=64, C=32), UNSUPPORTED),
    (dict(q=ctypes.c_void_p(P[0].value + 4)), INVALID),     # misaligned
    (dict(out=P[0]), INVALID),                                # out aliases q
    (dict(out=ctypes.c_void_p(P[2].value + 16)), INVALID),   # out overlaps v
    (dict(T=100000, wsb=16), WORKSPACE),                      # workspace too small
    (dict(T=100000, ws=NULL), WORKSPACE),                     # workspace missing
    (dict(T=100000, ws=P[3]), INVALID),                       # workspace overlaps out
])
def test_forward_error_paths(kw, status):
    assert fwd(**kw) == status


def fwd_noalloc(q=P[0], k=P[1], v=P[2], out=P[3], B=1, H=1, T=64, d=16, dv=16, C=32, eps=1e-6,
                dt=BF16, scan=0, stream=None):
    return am.lib().kata_forward_chunked_noalloc(q, k, v, out, B, H, T, d, dv, C, eps, dt, scan, stream)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), INVALID), (dict(out=NULL), INVALID), (dict(B=0), INVALID), (dict(T=0), INVALID),
    (dict(d=24), UNSUPPORTED), (dict(dv=48), UNSUPPORTED), (dict(C=16), UNSUPPORTED),
    (dict(eps=float("nan")), INVALID), (dict(dt=7), INVALID), (dict(scan=5), INVALID),
    (dict(q=ctypes.c_void_p(P[0].value + 4)), INVALID),
    (dict(out=P[0]), INVALID), (dict(out=ctypes.c_void_p(P[2].value + 16)), INVALID),
    # the fp32 forward of 8 heads of T = 131072 at d = 32 needs 67 MiB
    (dict(B=1, H=8, T=131072, d=32, dv=64, C=64, dt=F32), WORKSPACE),
])
def test_forward_noalloc_error_paths(kw, status):
    assert fwd_noalloc(**kw) == status


def test_forward_noalloc_scratch_limit():
    L = am.lib()
    assert am.KATA_NOALLOC_SCRATCH_BYTES == 64 << 20
    # the benchmarked bf16 forwards fit the scratch; the rejected fp32 shape above does not
    for (B, H, T, d, C) in [(4, 8, 2048, 16, 64), (2, 16, 8192, 32, 64), (1, 8, 131072, 16, 128)]:
        for scan in (0, 1, 2):
            plan = dict(kv.split("=") for kv in am.kata_forward_plan(B, H, T, d, 64, C, BF16, scan).split())
            assert 0 < int(plan["workspace_bytes"]) <= am.KATA_NOALLOC_SCRATCH_BYTES
    plan = dict(kv.split("=") for kv in am.kata_forward_plan(1, 8, 131072, 32, 64, 64, F32, 0).split())
    assert int(plan["workspace_bytes"]) > am.KATA_NOALLOC_SCRATCH_BYTES


def test_decode_error_paths():
    L = am.lib()
    dec = lambda S=P[0], z=P[1], q=P[2], k=P[3], v=P[4], out=P[5], B=1, H=1, d=16, dv=64, eps=1e-6, dt=F32: \
        L.kata_decode_step(S, z, q, k, v, out, B, H, d, dv, eps, dt, None)
    assert dec(S=NULL) == INVALID
    assert dec(out=NULL) == INVALID
    assert dec(B=0) == INVALID
    assert dec(d=8) == UNSUPPORTED
    assert dec(dv=100) == UNSUPPORTED
    assert dec(eps=-1.0) == INVALID
    assert dec(out=P[0]) == INVALID           # out aliases S
    assert dec(z=P[0]) == INVALID             # z aliases S
    assert dec(q=ctypes.c_void_p(P[2].value + 8)) == INVALID
    assert dec(dt=3) == INVALID


def test_prefill_and_feature_map_error_paths():
    L = am.lib()
    assert L.kata_prefill_state(NULL, P[1], P[2], P[3], 1, 1, 8, 16, 16, F32, None) == INVALID
    assert L.kata_prefill_state(P[0], P[1], P[2], P[3], 1, 1, 0, 16, 16, F32, None) == INVALID
    assert L.kata_prefill_state(P[0], P[1], P[2], P[3], 1, 1, 8, 12, 16, F32, None) == UNSUPPORTED
    assert L.kata_prefill_state(P[0], P[1], P[2], P[2], 1, 1, 8, 16, 16, F32, None) == INVALID
    assert L.kata_feature_map(NULL, P[1], 4, 16, F32, F32, None) == INVALID
    assert L.kata_feature_map(P[0], P[1], 0, 16, F32, F32, None) == INVALID
    assert L.kata_feature_map(P[0], P[1], 4, 65, F32, F32, None) == UNSUPPORTED
    assert L.kata_feature_map(P[0], P[0], 4, 16, F32, F32, None) == INVALID
    buf = ctypes.create_string_buffer(8)
    assert L.kata_forward_plan(1, 1, 64, 16, 16, 32, BF16, 0, None, 0) == INVALID
    assert L.kata_forward_plan(1, 1, 64, 16, 16, 32, BF16, 0, buf, 8) == OK
    assert len(buf.value) == 7  # truncated, NUL-terminated


def quad(q=P[0], k=P[1], v=P[2], out=P[3], B=1, H=1, T=300, d=16, dv=64, g=1, eps=1e-6, dt=BF16):
    return am.lib().kata_forward_quadratic(q, k, v, out, B, H, T, d, dv, g, eps, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), INVALID), (dict(out=NULL), INVALID),
    (dict(B=0), INVALID), (dict(T=0), INVALID), (dict(d=0), INVALID),
    (dict(dt=F32), UNSUPPORTED), (dict(d=24), UNSUPPORTED), (dict(dv=32), UNSUPPORTED),
    (dict(eps=-1.0), INVALID), (dict(eps=float("nan")), INVALID), (dict(dt=9), INVALID),
    (dict(k=ctypes.c_void_p(P[1].value + 2)), INVALID),      # misaligned
    (dict(out=P[1]), INVALID),                                # out aliases k
    (dict(out=ctypes.c_void_p(P[2].value + 64)), INVALID),   # out overlaps v
    (dict(B=1 << 20, H=1 << 10, T=1 << 20), UNSUPPORTED),     # grid too large
    (dict(g=0), INVALID), (dict(g=-2), INVALID), (dict(d=64, g=3), INVALID),  # g must divide d
    (dict(d=16, g=2), UNSUPPORTED), (dict(d=64, g=8), UNSUPPORTED),  # block width 8
    (dict(d=48, g=3), UNSUPPORTED), (dict(d=128, g=2), UNSUPPORTED),
])
def test_quadratic_error_paths(kw, status):
    assert quad(**kw) == status


def lin(q=P[0], k=P[1], v=P[2], out=P[3], B=1, H=1, T=300, d=64, dv=64, chunk=64, feat=0, shift=1e-6,
        eps=1e-6, dt=BF16, scan=0, ws=None, wsb=0):
    return am.lib().kata_forward_linear(q, k, v, out, B, H, T, d, dv, chunk, feat, shift, eps, dt, scan, ws,
                                        wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), INVALID), (dict(v=NULL), INVALID), (dict(B=0), INVALID), (dict(T=-1), INVALID),
    (dict(feat=3), INVALID), (dict(feat=-1), INVALID), (dict(dt=7), INVALID), (dict(scan=3), INVALID),
    (dict(dt=F32), UNSUPPORTED), (dict(d=32), UNSUPPORTED), (dict(dv=32), UNSUPPORTED),
    (dict(chunk=16), UNSUPPORTED), (dict(chunk=256), UNSUPPORTED), (dict(chunk=96), UNSUPPORTED),
    (dict(feat=2, chunk=48), UNSUPPORTED),
    (dict(shift=-1.0), INVALID), (dict(shift=float("inf")), INVALID), (dict(eps=float("nan")), INVALID),
    (dict(out=ctypes.c_void_p(P[3].value + 8)), INVALID),  # misaligned
    (dict(out=P[0]), INVALID),                              # out aliases q
    (dict(T=1 << 20), WORKSPACE),                           # several spans, no workspace
])
def test_linear_error_paths(kw, status):
    assert lin(**kw) == status


def test_linear_workspace_sizes():
    L = am.lib()
    # one span per head: no workspace
    assert L.kata_forward_linear_workspace_bytes(64, 16, 64, 64, 64, 64) == 0
    # B=1, H=16, T=131072: 2048 chunks per head in 32 spans of 64 chunks
    n = L.kata_forward_linear_workspace_bytes(1, 16, 131072, 64, 64, 64)
    assert n == 16 * 32 * 4 * 5 * 256 * 4
    assert L.kata_forward_linear_workspace_bytes(1, 16, 131072, 32, 64, 64) == 0  # unsupported
    # chunk 128: 1024 chunks per head in 32 spans of 32; chunk 32: 4096 in 32 spans of 128
    assert L.kata_forward_linear_workspace_bytes(1, 16, 131072, 64, 64, 128) == n
    assert L.kata_forward_linear_workspace_bytes(1, 16, 131072, 64, 64, 32) == n
    # B = 4, H = 12, T = 1024, chunk 32: 32 chunks in 11 spans of 3
    assert L.kata_forward_linear_workspace_bytes(4, 12, 1024, 64, 64, 32) == 48 * 11 * 4 * 5 * 256 * 4


def gated(q=P[0], k=P[1], v=P[2], lg=P[4], out=P[3], B=1, H=1, T=300, d=16, dv=64, chunk=128, dt=BF16,
          ws=P[5], wsb=1 << 30):
    return am.lib().kata_forward_gated(q, k, v, lg, out, B, H, T, d, dv, chunk, dt, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), INVALID), (dict(lg=NULL), INVALID), (dict(out=NULL), INVALID), (dict(H=0), INVALID),
    (dict(dt=5), INVALID), (dict(dt=F32), UNSUPPORTED), (dict(d=64), UNSUPPORTED), (dict(dv=16), UNSUPPORTED),
    (dict(chunk=32), UNSUPPORTED),
    (dict(lg=ctypes.c_void_p(P[4].value + 4)), INVALID),   # misaligned
    (dict(out=P[4]), INVALID),                              # out overlaps log_gamma
    (dict(ws=NULL, wsb=0), WORKSPACE), (dict(wsb=64), WORKSPACE),
    (dict(ws=P[3]), INVALID),                               # workspace overlaps out
])
def test_gated_error_paths(kw, status):
    assert gated(**kw) == status


def test_gated_workspace_sizes():
    L = am.lib()
    # T = 300, chunk 128: 3 chunks in 3 spans.  Span states (9 feature tiles x
    # 4 value tiles x 256 floats + 9 x 16 floats of z each), then the gate sums
    # and the key factors (300 floats each) and the chunk totals (3 floats),
    # each 256-byte aligned
    states = 3 * (9 * 4 * 256 + 9 * 16) * 4
    gb_off = (states + 255) // 256 * 256
    gk_off = (gb_off + 300 * 4 + 255) // 256 * 256
    ctot_off = (gk_off + 300 * 4 + 255) // 256 * 256
    assert L.kata_forward_gated_workspace_bytes(1, 1, 300, 16, 64, 128) == ctot_off + 3 * 4
    # 64 heads of one chunk: a single span, no states
    assert L.kata_forward_gated_workspace_bytes(8, 8, 100, 16, 64, 128) == 2 * 25600 + 64 * 4
    # d = 32: 33 feature tiles per span state (3 spans of one chunk)
    states = 3 * (33 * 4 * 256 + 33 * 16) * 4
    gb_off = (states + 255) // 256 * 256
    gk_off = (gb_off + 300 * 4 + 255) // 256 * 256
    ctot_off = (gk_off + 300 * 4 + 255) // 256 * 256
    assert L.kata_forward_gated_workspace_bytes(1, 1, 300, 32, 64, 128) == ctot_off + 3 * 4
    assert L.kata_forward_gated_workspace_bytes(1, 1, 300, 64, 64, 128) == 0  # unsupported


def test_gated_prefill_error_paths():
    L = am.lib()
    pre = lambda k=P[0], v=P[1], lg=P[2], S=P[3], B=1, H=1, T=10, d=16, dv=64, dt=F32: \
        L.kata_prefill_state_gated(k, v, lg, S, B, H, T, d, dv, dt, None)
    assert pre(k=NULL) == INVALID
    assert pre(lg=NULL) == INVALID
    assert pre(S=NULL) == INVALID
    assert pre(T=0) == INVALID
    assert pre(dt=4) == INVALID
    assert pre(d=24) == UNSUPPORTED
    assert pre(dv=48) == UNSUPPORTED
    assert pre(lg=ctypes.c_void_p(P[2].value + 2)) == INVALID   # misaligned
    assert pre(S=P[1]) == INVALID                               # S overlaps v
    assert pre(S=ctypes.c_void_p(P[2].value + 16)) == INVALID   # S overlaps log_gamma


def test_gated_decode_error_paths():
    L = am.lib()

    def step(S=P[0], q=P[1], k=P[2], v=P[3], lg=P[4], out=P[5], B=2, H=3, d=16, dv=64, dt=F32):
        return L.kata_decode_step_gated(S, q, k, v, lg, out, B, H, d, dv, dt, None)

    assert step(S=NULL) == INVALID
    assert step(lg=NULL) == INVALID
    assert step(B=0) == INVALID
    assert step(dt=4) == INVALID
    assert step(d=24) == UNSUPPORTED
    assert step(dv=48) == UNSUPPORTED
    assert step(lg=ctypes.c_void_p(P[4].value + 2)) == INVALID  # not 4-byte aligned
    assert step(out=P[4]) == INVALID                            # out overlaps log_gamma
    assert step(out=P[0]) == INVALID                            # out overlaps S



def blk(q=P[0], k=P[1], v=P[2], out=P[3], B=1, H=2, T=300, d=64, dv=64, g=4, chunk=64, eps=1e-6, dt=BF16,
        scan=0, ws=P[5], wsb=1 << 30):
    return am.lib().kata_forward_chunked_blocks(q, k, v, out, B, H, T, d, dv, g, chunk, eps, dt, scan, ws, wsb,
                                                None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), INVALID), (dict(B=0), INVALID), (dict(g=0), INVALID), (dict(g=3), INVALID),
    (dict(scan=9), INVALID), (dict(dt=3), INVALID), (dict(eps=-1.0), INVALID),
    (dict(dt=F32), UNSUPPORTED), (dict(g=8), UNSUPPORTED), (dict(chunk=128), UNSUPPORTED),
    (dict(d=32, g=2), UNSUPPORTED), (dict(dv=32), UNSUPPORTED), (dict(g=2, chunk=128), UNSUPPORTED),
    (dict(out=P[1]), INVALID), (dict(ws=NULL, wsb=0, T=1 << 16), WORKSPACE),
    (dict(g=1, d=24), UNSUPPORTED),   # g = 1 takes kata_forward_chunked's checks
])
def test_chunked_blocks_error_paths(kw, status):
    assert blk(**kw) == status


def test_chunked_blocks_workspace():
    L = am.lib()
    # g = 1 is kata_forward_chunked's workspace
    assert (L.kata_forward_chunked_blocks_workspace_bytes(1, 8, 131072, 16, 64, 1, 128, 0)
            == L.kata_forward_workspace_bytes(1, 8, 131072, 16, 64, 128, 0))
    # KATA-M4: 34 feature tiles x (4 x 256 + 16) floats per span state
    E = (34 * 4 * 256 + 34 * 16) * 4
    n4 = L.kata_forward_chunked_blocks_workspace_bytes(8, 16, 16384, 64, 64, 4, 64, 0)
    assert n4 > 0 and n4 % E == 0
    # KATA-M2 / M1: 2 / 4 slices of span states, then fp32 partial reads
    # (68 floats per token-head), 256-byte aligned
    part = 8 * 16 * 16384 * 68 * 4
    for g, nsl in ((2, 2), (1, 4)):
        n = L.kata_forward_chunked_blocks_workspace_bytes(8, 16, 16384, 64, 64, g, 64, 0)
        assert n == (nsl * n4 + 255) // 256 * 256 + part
    assert L.kata_forward_chunked_blocks_workspace_bytes(8, 16, 16384, 64, 64, 8, 64, 0) == 0


def test_probe_rejects_bad_arguments():
    # every rejection happens before any launch
    L = am.lib()
    assert L.kata_probe_mfma_bf16(None, 8, 100, None) == -1
    assert L.kata_probe_mfma_bf16(8, 8, 100, None) == -1          # misaligned sink
    assert L.kata_probe_mfma_bf16(256, 0, 100, None) == -1        # no workgroups
    assert L.kata_probe_mfma_bf16(256, 8, 0, None) == -1          # no rounds
    assert L.kata_probe_mfma_bf16(256, (1 << 20) + 1, 1, None) == -1
    assert L.kata_probe_mfma_bf16(256, 1, (1 << 24) + 1, None) == -1


def test_recompute_plan():
    """Scan 3: no span sums, no prefix, no workspace; every chunk of a head
    belongs to exactly one readout workgroup's span."""
    L = am.lib()
    for (B, H, T, C) in [(4, 8, 2048, 64), (4, 8, 2048, 128), (1, 2, 77, 128), (1, 3, 40000, 128),
                         (1, 8, 131072, 128)]:
        assert L.kata_forward_workspace_bytes(B, H, T, 16, 64, C, 3) == 0
        plan = am.kata_forward_plan(B, H, T, 16, 64, C, BF16, "recompute")
        f = dict(kv.split("=") for kv in plan.split())
        assert f["scan"] == "recompute" and f["wg_state"] == "0" and f["workspace_bytes"] == "0"
        G, n_spans, n_chunks = int(f["chunks_per_span"]), int(f["n_spans"]), int(f["n_chunks"])
        assert n_chunks == -(-T // C) and G * n_spans >= n_chunks > G * (n_spans - 1)
        assert int(f["wg_output"]) == B * H * n_spans and f["paired_even_span"] == "0"
    # the other forwards take no scan 3
    assert L.kata_forward_workspace_bytes(1, 1, 64, 32, 64, 64, 3) == 0
    assert L.kata_forward_chunked_blocks_workspace_bytes(1, 1, 64, 64, 64, 4, 64, 3) == 0


def test_fused_plan():
    """Scan 4: span sums stored unscanned, no prefix launch, the workspace of
    the sequential plan; the automatic choice at d = 16 up to 16 spans per
    head, without paired spans."""
    L = am.lib()
    for (B, H, T, C) in [(4, 8, 2048, 64), (4, 8, 2048, 128), (4, 8, 4096, 64), (8, 8, 2048, 64)]:
        plan = am.kata_forward_plan(B, H, T, 16, 64, C, BF16, "auto")
        f = dict(kv.split("=") for kv in plan.split())
        assert f["scan"] == "fused" and f["paired_even_span"] == "0", plan
        assert 1 < int(f["n_spans"]) <= 16
        assert int(f["wg_state"]) == B * H * (int(f["n_spans"]) - 1)
        assert L.kata_forward_workspace_bytes(B, H, T, 16, 64, C, 0) == \
            L.kata_forward_workspace_bytes(B, H, T, 16, 64, C, 1) == \
            L.kata_forward_workspace_bytes(B, H, T, 16, 64, C, 4) > 0
    for (B, H, T, C) in [(1, 8, 131072, 128), (2, 8, 8192, 64)]:
        auto = dict(kv.split("=") for kv in am.kata_forward_plan(B, H, T, 16, 64, C, BF16, "auto").split())
        assert auto["scan"] == "sequential" and int(auto["n_spans"]) > 16
        fused = dict(kv.split("=") for kv in am.kata_forward_plan(B, H, T, 16, 64, C, BF16, "fused").split())
        assert fused["scan"] == "fused" and fused["paired_even_span"] == "0"
        assert fused["n_spans"] == auto["n_spans"] and fused["workspace_bytes"] == auto["workspace_bytes"]
    # few heads at short T: 16 spans of at most 256 tokens in place of more spans and a prefix launch
    for (B, H, T, C, n_seq) in [(2, 8, 2048, 64, 32), (1, 8, 4096, 64, 64), (1, 1, 2048, 64, 32)]:
        auto = dict(kv.split("=") for kv in am.kata_forward_plan(B, H, T, 16, 64, C, BF16, "auto").split())
        seq = dict(kv.split("=") for kv in am.kata_forward_plan(B, H, T, 16, 64, C, BF16, "sequential").split())
        assert auto["scan"] == "fused" and auto["n_spans"] == "16", auto
        assert int(auto["chunks_per_span"]) * C <= 256
        assert seq["n_spans"] == str(n_seq)
        assert L.kata_forward_workspace_bytes(B, H, T, 16, 64, C, 0) < L.kata_forward_workspace_bytes(B, H, T, 16, 64, C, 1)
    assert "scan=sequential" in am.kata_forward_plan(1, 8, 8192, 16, 64, 128, BF16, "auto")
    # d = 32 (chunk 64) takes it up to 4 spans per head
    for (B, H, T, n) in [(8, 16, 2048, 2), (4, 16, 4096, 4)]:
        f = dict(kv.split("=") for kv in am.kata_forward_plan(B, H, T, 32, 64, 64, BF16, "auto").split())
        assert f["scan"] == "fused" and f["n_spans"] == str(n)
    assert "scan=fused" in am.kata_forward_plan(2, 16, 8192, 32, 64, 64, BF16, "fused")
    # d = 32 at 8 spans per head, fp32 and the block maps keep their prefix launch
    assert "scan=sequential" in am.kata_forward_plan(2, 16, 8192, 32, 64, 64, BF16, "auto")
    assert "scan=fused" not in am.kata_forward_plan(4, 8, 2048, 16, 64, 64, F32, "auto")
    assert L.kata_forward_chunked_blocks_workspace_bytes(1, 1, 64, 64, 64, 4, 64, 4) == 0

#!/usr/bin/env python3
"""Benchmark of libkata on one MI355X.

A step is one chunked forward (feature map, intra-chunk block, span states,
prefix over spans, readout -- the whole forward path) over the long-context
workload B=1, H=8, T=131072, d=16, dv=64, chunk=128, bf16, with inputs already
resident in HBM.  `value` is sequence tokens per second, B*T / t_step.  Both
prefix variants (sequential and associative) are timed and reported; `value`
is the library's default (auto) choice.  The recurrent decode workload
(4096 heads, D=136, dv=64, fp32 state, 1024 steps) is timed in the same run
and reported under "decode" with its own roofline: the eager launch loop, the
kernel alone, and the loop captured in one HIP graph.  The same decode over
512 sequences (290 MB of state, beyond the 256 MB Infinity Cache) is reported
under "decode_beyond_cache".  "attainable" gives the whole step against the
larger of its HBM time (minimal bytes) and its MFMA time (useful FLOPs).

The fp64 oracle's timing on the host is reported as cpu_baseline: its chunked
form over the whole T = 131072 workload, with the plain definition on one head
and per-workload timings beside it.  A baseline, not the target.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--warmup-ms MS] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--warmup-ms", type=float, default=200.0,
                    help="untimed warm-up continues past --warmup calls until this much wall time "
                         "has passed, so the timed regions start at the clocks the GPU holds under load")
    ap.add_argument("--repeats", type=int, default=5,
                    help="interleaved timed regions of K steps per prefix variant (median reported)")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-captured decode timing")
    ap.add_argument("--no-other", action="store_true", help="skip the other forward workloads")
    ap.add_argument("--no-linear", action="store_true", help="skip the linear-feature timings")
    ap.add_argument("--no-gated", action="store_true", help="skip the gated-read timings")
    ap.add_argument("--no-table8", action="store_true",
                    help="skip the quadratic block-map timings on the d = 64 shape")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    ap.add_argument("--calib-read", action="store_true",
                    help="only run a read-only reduction of known size (second counter calibration)")
    return ap.parse_args()


# ------------------------------------------------------------------ HIP events

class Hip:
    """Minimal HIP runtime access for events on the stream the library uses."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.h.hipEventRecord(e, stream) == 0

    def ms(self, a, b) -> float:
        out = ctypes.c_float()
        assert self.h.hipEventSynchronize(b) == 0
        assert self.h.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return float(out.value)

    def destroy(self, e):
        self.h.hipEventDestroy(e)


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "associative_memory_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
    except Exception:
        return None
    e = t.get(kernel_key)
    if not e or e.get("source_hash") != source_hash():
        return None
    return e.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ measured peaks

def measure_peaks(hip, am, torch):
    """The datasheet peaks re-measured on this device: the dense bf16
    matrix-core rate from the library's probe (independent 16x16x32 product
    chains, 8 waves per SIMD) and the HBM bandwidth of a 1 GiB
    device-to-device copy (bytes read + written), each the best of 5 timed
    launches after 2 warm-ups."""
    stream = torch.cuda.current_stream().cuda_stream
    wgs, iters = 2048, 5000  # 8 waves per SIMD
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")

    def best(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = hip.event(), hip.event()
            hip.record(e0, stream)
            fn()
            hip.record(e1, stream)
            ts.append(hip.ms(e0, e1) * 1e-3)
            hip.destroy(e0)
            hip.destroy(e1)
        return min(ts)

    flops = am.kata_probe_mfma_bf16(sink, wgs, iters)
    t_mfma = best(lambda: am.kata_probe_mfma_bf16(sink, wgs, iters))
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_copy = best(lambda: dst.copy_(src))
    del src, dst, sink
    return {"mfma_bf16_tflops": round(flops / t_mfma / 1e12, 1),
            "mfma_bf16_datasheet_tflops": BF16_PEAK_TFLOPS,
            "hbm_copy_gbs": round(2 * n / t_copy / 1e9, 1),
            "hbm_datasheet_gbs": HBM_PEAK_GBS,
            "method": "matrix cores: kata_probe_mfma_bf16, 2048 workgroups x 4 waves x 8 independent "
                      "16x16x32 bf16 chains x 5000 rounds; HBM: 1 GiB device-to-device copy, read + "
                      "write bytes; best of 5 after 2 warm-ups"}


# ------------------------------------------------------------------ forward

def bench_forward(args, hip, am, ki, torch):
    """The T = 131072 forward with each prefix variant (sequential,
    associative, auto).  The variants are timed interleaved: `repeats`
    rounds, each running every variant once (the order rotating from round to
    round) as a region of exactly K forwards between events on the library's
    stream; a variant's figure is the median over its regions.  Per-stage
    kernel durations come from a separate pass of K profiled forwards per
    variant (median per stage)."""
    w = ki.LONG
    inp = ki.workload_inputs(w)

    def dev(a):
        return torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()

    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    out = torch.empty((w.B, w.H, w.T, w.dv), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    scans = ("sequential", "associative", "auto")
    ws = {}
    for scan in scans:
        ws_bytes = am.kata_forward_workspace_bytes(w.B, w.H, w.T, w.d, w.dv, w.chunk, scan)
        ws[scan] = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    _warm(args, torch, *[
        (lambda sc=scan: am.kata_forward_chunked(q, k, v, w.chunk, eps=w.eps, scan=sc, out=out,
                                                 workspace=ws[sc])) for scan in scans])
    samples = {scan: [] for scan in scans}
    walls = {scan: [] for scan in scans}
    for r in range(args.repeats):
        for i in range(len(scans)):
            scan = scans[(r + i) % len(scans)]
            e0, e1 = hip.event(), hip.event()
            torch.cuda.synchronize()
            t_wall = time.perf_counter()
            hip.record(e0, stream)
            for _ in range(args.steps):
                am.kata_forward_chunked(q, k, v, w.chunk, eps=w.eps, scan=scan, out=out, workspace=ws[scan])
            hip.record(e1, stream)
            torch.cuda.synchronize()
            walls[scan].append(1e3 * (time.perf_counter() - t_wall) / args.steps)
            samples[scan].append(hip.ms(e0, e1) / args.steps)
            hip.destroy(e0)
            hip.destroy(e1)
    results = {}
    for scan in scans:
        # per-stage kernel durations, same launches, one event set per step
        sets = []
        for _ in range(args.steps):
            ev = am.StageEvents()
            hs = [hip.event() for _ in range(6)]
            for i in range(3):
                ev.stage_begin[i] = hs[2 * i]
                ev.stage_end[i] = hs[2 * i + 1]
            am.kata_forward_chunked_profiled(q, k, v, w.chunk, ev, eps=w.eps, scan=scan, out=out,
                                             workspace=ws[scan])
            sets.append(hs)
        torch.cuda.synchronize()
        per_stage = [[], [], []]
        for hs in sets:
            for i in range(3):
                per_stage[i].append(hip.ms(hs[2 * i], hs[2 * i + 1]))
            for h in hs:
                hip.destroy(h)
        stage_ms = [statistics.median(x) for x in per_stage]
        ms_step = statistics.median(samples[scan])
        results[scan] = {
            "ms_per_step": ms_step,
            "ms_per_step_samples": [round(x, 5) for x in samples[scan]],
            "wall_ms_per_step": statistics.median(walls[scan]),
            "tokens_per_s": w.B * w.T / (ms_step * 1e-3),
            "stage_ms": {"span_states": stage_ms[0], "prefix": stage_ms[1], "readout": stage_ms[2]},
            "plan": am.kata_forward_plan(w.B, w.H, w.T, w.d, w.dv, w.chunk, am.KATA_BF16, scan),
        }
    del ws
    return w, inp, results


def _warm(args, torch, *fns):
    """Untimed warm-up: every callable in turn, at least `warmup` rounds and
    until `warmup_ms` of wall time has passed (the GPU leaves its idle clocks
    over tens of milliseconds of work; a handful of calls does not get it
    there)."""
    t0 = time.perf_counter()
    rounds = 0
    while rounds < args.warmup or 1e3 * (time.perf_counter() - t0) < args.warmup_ms:
        for f in fns:
            f()
        rounds += 1
        if rounds % 8 == 0 or rounds >= args.warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def _interleaved_ms(args, hip, torch, calls):
    """Median milliseconds per call of each named callable: after the warm-up
    (`_warm`), `repeats` rounds each time `steps` back-to-back calls of
    every callable (HIP events on the current stream), the order rotated per
    round so no variant always runs first."""
    stream = torch.cuda.current_stream().cuda_stream
    names = list(calls)
    _warm(args, torch, *calls.values())
    samples = {n: [] for n in names}
    for r in range(args.repeats):
        shift = r % len(names)
        for n in names[shift:] + names[:shift]:
            e0, e1 = hip.event(), hip.event()
            hip.record(e0, stream)
            for _ in range(args.steps):
                calls[n]()
            hip.record(e1, stream)
            torch.cuda.synchronize()
            samples[n].append(hip.ms(e0, e1) / args.steps)
            hip.destroy(e0)
            hip.destroy(e1)
    return {n: (statistics.median(x), x) for n, x in samples.items()}


def res_plan(am, ki, w):
    """The library's plan string for workload w (AUTO prefix)."""
    return am.kata_forward_plan(w.B, w.H, w.T, w.d, w.dv, w.chunk,
                                am.KATA_BF16 if w.dtype == ki.BF16 else am.KATA_F32, "auto")


def bench_other_workloads(args, hip, am, ki, torch):
    """The other forward workloads (parity-test shapes), library default plan,
    timed interleaved with the quadratic form and (d = 16) the plan that forms
    the prefix in the readout."""
    res = {}
    for w in (ki.MEDIUM, ki.WIDE, ki.TINY):
        inp = ki.workload_inputs(w)
        if w.dtype == ki.BF16:
            dev = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()
        else:
            dev = lambda a: torch.from_numpy(a).cuda()
        q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
        out = torch.empty((w.B, w.H, w.T, w.dv), dtype=q.dtype, device="cuda")
        ws_bytes = am.kata_forward_workspace_bytes(w.B, w.H, w.T, w.d, w.dv, w.chunk, "auto")
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        calls = {"chunked": lambda: am.kata_forward_chunked(q, k, v, w.chunk, eps=w.eps, out=out, workspace=ws)}
        quad = w.dtype == ki.BF16 and w.dv == 64
        rc = w.dtype == ki.BF16 and w.d == 16 and w.dv == 64
        if quad:
            calls["quadratic"] = lambda: am.kata_forward_quadratic(q, k, v, eps=w.eps, g=w.g, out=out)
        if rc:
            # the prefix formed inside the readout workgroups (one launch, no workspace)
            calls["recompute"] = lambda: am.kata_forward_chunked(q, k, v, w.chunk, eps=w.eps, scan="recompute", out=out)
        if w.dtype == ki.BF16 and "scan=sequential" not in res_plan(am, ki, w):
            # the three-launch plan beside the library's choice
            calls["sequential"] = lambda: am.kata_forward_chunked(q, k, v, w.chunk, eps=w.eps, scan="sequential",
                                                                  out=out, workspace=ws)
        t = _interleaved_ms(args, hip, torch, calls)
        ms = t["chunked"][0]
        D = w.d * (w.d + 1) // 2
        BHT = w.B * w.H * w.T
        es = 2 if w.dtype == ki.BF16 else 4
        flops = 2 * ((w.chunk + 1) / 2 * (w.d + w.dv) + 2 * D * w.dv + 2 * D) * BHT
        bytes_ = (es * (2 * w.d + w.dv) + es * w.dv) * BHT
        res[w.name] = {
            "ms_per_step": round(ms, 4),
            "ms_per_step_samples": [round(x, 5) for x in t["chunked"][1]],
            "tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1),
            "useful_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "hbm_gbs": round(bytes_ / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(bytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "plan": am.kata_forward_plan(w.B, w.H, w.T, w.d, w.dv, w.chunk,
                                         am.KATA_BF16 if w.dtype == ki.BF16 else am.KATA_F32, "auto"),
        }
        if quad:
            qms = t["quadratic"][0]
            qflops = 2 * (w.T + 1) / 2 * (w.d + w.dv) * w.B * w.H * w.T
            res[w.name]["quadratic"] = {
                "ms_per_step": round(qms, 4), "tokens_per_s": round(w.B * w.T / (qms * 1e-3), 1),
                "useful_tflops": round(qflops / (qms * 1e-3) / 1e12, 2),
                "mfma_frac": round(qflops / (qms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        if "sequential" in t:
            sms = t["sequential"][0]
            res[w.name]["sequential"] = {
                "ms_per_step": round(sms, 4),
                "tokens_per_s": round(w.B * w.T / (sms * 1e-3), 1),
                "plan": am.kata_forward_plan(w.B, w.H, w.T, w.d, w.dv, w.chunk, am.KATA_BF16, "sequential"),
            }
        if rc:
            rms = t["recompute"][0]
            res[w.name]["recompute"] = {
                "ms_per_step": round(rms, 4),
                "tokens_per_s": round(w.B * w.T / (rms * 1e-3), 1),
                "plan": am.kata_forward_plan(w.B, w.H, w.T, w.d, w.dv, w.chunk, am.KATA_BF16, "recompute"),
            }
    return res


def bench_quadratic(args, hip, am, torch, w, q, k, v, out):
    """The direct O(T^2) form on the same inputs.  Useful FLOPs: the causal
    triangle of (d + dv)-wide products, 2 * (T+1)/2 * (d + dv) per
    token-head as for the intra-chunk block, with the chunk as long as the
    sequence (the KATA-Mg score costs the same 2d per pair for any g)."""
    stream = torch.cuda.current_stream().cuda_stream
    _warm(args, torch, lambda: am.kata_forward_quadratic(q, k, v, eps=w.eps, g=w.g, out=out))
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(args.steps):
        am.kata_forward_quadratic(q, k, v, eps=w.eps, g=w.g, out=out)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    ms = hip.ms(e0, e1) / args.steps
    hip.destroy(e0)
    hip.destroy(e1)
    flops = 2 * (w.T + 1) / 2 * (w.d + w.dv) * w.B * w.H * w.T
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1),
            "useful_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}


# forward latency of the quadratic KATA-M1 / KATA-M2 kernels on one H100, in
# ms, from Table 8 of the KATA page (B = 8, H = 16, d_head = 64, bf16):
# context for the same shapes here, not a target on this hardware
PAGE_TABLE8_QUAD_MS = {(1024, 1): 0.07, (4096, 1): 0.58, (16384, 1): 8.92,
                       (1024, 2): 0.07, (4096, 2): 0.72, (16384, 2): 10.62}
# the page's linear-state (O(T)) KATA-M1 / KATA-M2 kernels on the same shape
PAGE_TABLE8_LINEAR_MS = {(1024, 1): 2.68, (4096, 1): 10.34, (16384, 1): 41.14, (131072, 1): 327.9,
                         (1024, 2): 0.68, (4096, 2): 2.70, (16384, 2): 10.68, (131072, 2): 85.66}


def bench_table8(args, hip, am, ki, torch):
    """The quadratic form with the KATA-Mg block maps (g = 1, 2, 4) on the
    page's Table 8 shape, inputs drawn on the device; and the chunked O(T)
    form of KATA-M4, KATA-M2 and KATA-M1 (g = 4, 2, 1; chunk 64) on the same
    shape up to T = 131072.  Chunked useful FLOPs: 2 [(C+1)/2 (d + dv) +
    2 D dv + 2 D] per token-head with D = 544, 1056, 2080 features."""
    res = {}
    for w in ki.TABLE8_QUAD:
        q, k, v = ki.forward_inputs_torch(w.B, w.H, w.T, w.d, w.dv, w.seed, "cuda")
        out = torch.empty_like(v)
        r = bench_quadratic(args, hip, am, torch, w, q, k, v, out)
        r["page_h100_ms"] = PAGE_TABLE8_QUAD_MS.get((w.T, w.g))
        res[w.name] = r
        del q, k, v, out
    stream = torch.cuda.current_stream().cuda_stream
    C = 64
    for T, g in ((T, g) for T in (1024, 4096, 16384, 131072) for g in (4, 2, 1)):
        D = {4: 4 * 136, 2: 2 * 528, 1: 2080}[g]
        w = ki.table8(T, g, 70)
        q, k, v = ki.forward_inputs_torch(w.B, w.H, w.T, w.d, w.dv, w.seed, "cuda")
        out = torch.empty_like(v)
        need = am.lib().kata_forward_chunked_blocks_workspace_bytes(w.B, w.H, w.T, w.d, w.dv, g, C, 0)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        _warm(args, torch, lambda: am.kata_forward_chunked_blocks(q, k, v, g, chunk=C, out=out, workspace=ws))
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, stream)
        for _ in range(args.steps):
            am.kata_forward_chunked_blocks(q, k, v, g, chunk=C, out=out, workspace=ws)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        ms = hip.ms(e0, e1) / args.steps
        hip.destroy(e0)
        hip.destroy(e1)
        flops = 2 * ((C + 1) / 2 * (w.d + w.dv) + 2 * D * w.dv + 2 * D) * w.B * w.H * w.T
        res[w.name.replace("_bf16", "_chunked_bf16")] = {
            "ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1),
            "useful_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "page_h100_ms": PAGE_TABLE8_LINEAR_MS.get((T, g))}
        del q, k, v, out, ws
    return res


# throughput of the page's first-order kernels on one H100, Mtok/s (context
# for the same shapes, not targets on this hardware):
# Table 11 -- B = 1, H = 16, d_head = 64, bf16, the identity feature
# psi(x) = x, chunk 128: its sequential linear-chunk kernel and its tree-scan
# kernel, by T;
PAGE_TABLE11_MTOKS = {2048: (6.7, 19.4), 4096: (13.6, 39.9), 8192: (23.4, 44.5), 16384: (24.1, 47.6),
                      32768: (24.9, 49.4), 65536: (25.5, 67.5), 131072: (25.8, 69.4)}
# App. E.1 -- B = 4, H = 12, dv = 64, chunk 32, orthant / Lorentz features:
# its linear (sequential) and tree (associative) kernels, by (T, feature)
PAGE_E1_MTOKS = {(1024, "orthant"): (24.1, 25.6), (1024, "lorentz"): (24.1, 25.6),
                 (2048, "orthant"): (27.3, 30.3), (2048, "lorentz"): (27.3, 30.3),
                 (4096, "orthant"): (29.8, 33.5)}


def _time_linear(args, hip, am, torch, q, k, v, out, ws, feature, chunk, scan):
    stream = torch.cuda.current_stream().cuda_stream
    _warm(args, torch, lambda: am.kata_forward_linear(q, k, v, feature=feature, chunk=chunk, scan=scan,
                                                      out=out, workspace=ws))
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(args.steps):
        am.kata_forward_linear(q, k, v, feature=feature, chunk=chunk, scan=scan, out=out, workspace=ws)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    ms = hip.ms(e0, e1) / args.steps
    hip.destroy(e0)
    hip.destroy(e1)
    return ms


def bench_linear(args, hip, am, ki, torch):
    """The linear-feature chunked forward (D = d = 64), both prefixes side by
    side: the identity map on the page's Table 11 slice (B = 1, H = 16,
    chunk 128, T = 2048 .. 131072) and the orthant / Lorentz maps on its
    App. E.1 shape (B = 4, H = 12, chunk 32, T = 1024 .. 4096) and at the
    Table 11 shape, inputs drawn on the device.  Algorithmic bytes: q, k, v
    read and out written once, 2 (2d + dv) + 2 dv = 512 B per token-head;
    useful FLOPs 2 [(C+1)/2 (d + dv) + 2 d dv (+ 2 d for the denominator)]
    per token-head."""
    res = {}
    d = dv = 64
    runs = [(1, 16, T, "identity", 128) for T in sorted(PAGE_TABLE11_MTOKS)]
    runs += [(4, 12, T, f, 32) for T in (1024, 2048, 4096) for f in ("orthant", "lorentz")]
    runs += [(1, 16, 131072, f, 128) for f in ("orthant", "lorentz")]
    for (B, H, T, feature, C) in runs:
        q, k, v = ki.forward_inputs_torch(B, H, T, d, dv, 80 + T % 97, "cuda")
        out = torch.empty_like(v)
        need = am.kata_forward_linear_workspace_bytes(B, H, T, d, dv, C)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        BHT = B * H * T
        bytes_ = (2 * (2 * d + dv) + 2 * dv) * BHT
        den = 0 if feature == "identity" else 2 * d
        flops = 2 * ((C + 1) / 2 * (d + dv) + 2 * d * dv + den) * BHT
        r = {}
        for scan in ("sequential", "associative"):
            ms = _time_linear(args, hip, am, torch, q, k, v, out, ws, feature, C, scan)
            r[scan] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
                       "hbm_frac": round(bytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "useful_tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
        r["assoc_over_seq"] = round(r["sequential"]["ms_per_step"] / r["associative"]["ms_per_step"], 3)
        if feature == "identity":
            page = PAGE_TABLE11_MTOKS.get(T)
            r["page_h100_mtoks"] = {"linear_chunk": page[0], "tree_scan": page[1],
                                    "source": "Table 11 (same shape, identity feature, chunk 128)"}
        elif C == 32:
            page = PAGE_E1_MTOKS.get((T, feature))
            if page:
                r["page_h100_mtoks"] = {"linear": page[0], "tree": page[1],
                                        "source": "App. E.1 table (same shape, same feature, chunk 32)"}
        res[f"B{B}_H{H}_T{T}_d64_dv64_{feature}_C{C}_bf16"] = r
        del q, k, v, out, ws
    return res


def bench_gated(args, hip, am, ki, torch):
    """The gated read (GatedKATA) on the T = 131072 and T = 2048 (d = 16)
    and T = 8192 (d = 32) forward shapes at both chunk lengths, gates from the
    seeded recipe.
    Algorithmic bytes: q, k, v, the fp32 gate read and out written,
    2 (2d + dv) + 4 + 2 dv = 324 B per token-head."""
    res = {}
    stream = torch.cuda.current_stream().cuda_stream
    for w in (ki.LONG, ki.MEDIUM, ki.WIDE):
        q, k, v = ki.forward_inputs_torch(w.B, w.H, w.T, w.d, w.dv, w.seed, "cuda")
        lg = torch.from_numpy(ki.draw_log_gamma(w.B, w.H, w.T, w.seed)).cuda()
        out = torch.empty_like(v)
        for C in (64, 128):
            need = am.kata_forward_gated_workspace_bytes(w.B, w.H, w.T, w.d, w.dv, C)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
            _warm(args, torch, lambda: am.kata_forward_gated(q, k, v, lg, chunk=C, out=out, workspace=ws))
            e0, e1 = hip.event(), hip.event()
            hip.record(e0, stream)
            for _ in range(args.steps):
                am.kata_forward_gated(q, k, v, lg, chunk=C, out=out, workspace=ws)
            hip.record(e1, stream)
            torch.cuda.synchronize()
            ms = hip.ms(e0, e1) / args.steps
            hip.destroy(e0)
            hip.destroy(e1)
            BHT = w.B * w.H * w.T
            bytes_ = (2 * (2 * w.d + w.dv) + 4 + 2 * w.dv) * BHT
            res[f"{w.name.replace('_C128', '').replace('_C64', '')}_gated_C{C}"] = {
                "ms_per_step": round(ms, 4),
                "tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1),
                "hbm_gbs": round(bytes_ / (ms * 1e-3) / 1e9, 1),
                "hbm_frac": round(bytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            }
            del ws
        del q, k, v, lg, out
    return res


# ------------------------------------------------------------------ decode

def bench_feature_map(args, hip, am, ki, torch):
    """The standalone feature map on the query rows of two forward workloads
    (bf16 in, bf16 out): HBM-bound, bytes = rows * (d + D) * 2."""
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for w in (ki.LONG, ki.WIDE):
        x = ki.forward_inputs_torch(w.B, w.H, w.T, w.d, w.dv, w.seed, "cuda")[0].reshape(-1, w.d)
        rows, D = x.shape[0], w.d * (w.d + 1) // 2
        phi = torch.empty((rows, D), dtype=torch.bfloat16, device="cuda")
        _warm(args, torch, lambda: am.kata_feature_map(x, out=phi))
        samples = []
        for _ in range(args.repeats):
            e0, e1 = hip.event(), hip.event()
            hip.record(e0, stream)
            for _ in range(args.steps):
                am.kata_feature_map(x, out=phi)
            hip.record(e1, stream)
            torch.cuda.synchronize()
            samples.append(hip.ms(e0, e1) / args.steps)
            hip.destroy(e0)
            hip.destroy(e1)
        ms = statistics.median(samples)
        nbytes = rows * (w.d + D) * 2
        res[f"rows{rows}_d{w.d}_bf16"] = {
            "ms_per_call": round(ms, 5), "ms_per_call_samples": [round(t, 5) for t in samples],
            "rows_per_s": round(rows / (ms * 1e-3), 1), "bytes_per_call": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
        del x, phi
    return res


def bench_decode(args, hip, am, ki, torch, w):
    """Recurrent decode: `steps` consecutive kata_decode_step launches over
    every head, timed three ways on the library's stream: the eager launch
    loop, each launch alone (kernel duration), and the whole loop captured in
    one HIP graph and replayed."""
    steps = args.decode_steps
    pk, pv, sq, sk, sv = ki.decode_inputs_torch(w.seed, w.heads, w.prefill, steps, w.d, w.dv, "cuda")
    S, z = am.kata_prefill_state(pk[:, None], pv[:, None])
    del pk, pv
    out = torch.empty((w.heads, w.dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    # warm-up steps on a copy of the state, so the timed loop starts from the prefill
    S_w, z_w = S.clone(), z.clone()
    _warm(args, torch, lambda: am.kata_decode_step(S_w, z_w, sq[0], sk[0], sv[0], eps=w.eps, out=out))
    del S_w, z_w
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for s in range(steps):
        am.kata_decode_step(S, z, sq[s], sk[s], sv[s], eps=w.eps, out=out)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    loop_ms = hip.ms(e0, e1)
    # per-launch kernel durations
    n = min(steps, 256)
    evs = [(hip.event(), hip.event()) for _ in range(n)]
    for s in range(n):
        hip.record(evs[s][0], stream)
        am.kata_decode_step(S, z, sq[s], sk[s], sv[s], eps=w.eps, out=out)
        hip.record(evs[s][1], stream)
    torch.cuda.synchronize()
    kern_ms = sum(hip.ms(a, b) for a, b in evs) / n
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    # the same loop captured in one graph (launch overhead removed)
    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for s in range(steps):
                    am.kata_decode_step(S, z, sq[s], sk[s], sv[s], eps=w.eps, out=out)
        torch.cuda.current_stream().wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        reps = 3
        hip.record(e0, stream)
        for _ in range(reps):
            g.replay()
        hip.record(e1, stream)
        torch.cuda.synchronize()
        graph_ms = hip.ms(e0, e1) / (reps * steps)
        del g
    hip.destroy(e0)
    hip.destroy(e1)
    D = w.d * (w.d + 1) // 2
    bytes_per_head = 2 * (D * w.dv + D) * 4 + (2 * w.d + 2 * w.dv) * 4
    alg_bytes = w.heads * bytes_per_head
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    state_mb = w.heads * (D * w.dv + D) * 4 / 1e6
    res = {
        "workload": w.name,
        "heads": w.heads,
        "steps": steps,
        "ms_per_step": loop_ms / steps,
        "kernel_ms": kern_ms,
        "graph_ms_per_step": graph_ms,
        "tokens_per_s": w.seqs * steps / (loop_ms * 1e-3),
        "head_tokens_per_s": w.heads * steps / (loop_ms * 1e-3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for("decode" if w is ki.DECODE else "decode_512"),
                     "algorithmic_bytes_per_launch": alg_bytes},
        "note": "state %.1f MB %s the 256 MB Infinity Cache" % (state_mb, "fits" if state_mb < 256 else "exceeds"),
    }
    if graph_ms:
        res["graph_tokens_per_s"] = w.seqs / (graph_ms * 1e-3)
        res["graph_roofline_frac"] = round(alg_bytes / (graph_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    del S, z, sq, sk, sv, out
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline(w, inp, ki):
    """The fp64 oracle timed on this host's cores: a baseline, not a target.

    value: the whole T = 131072 workload (all heads, every token) through the
    oracle's chunked form (Eqs. 17-20, the O(T) algorithm the device runs).
    Beside it: the plain O(T^2) definition on one head of that workload,
    scaled to all heads; the definition over the whole of each smaller
    forward workload; and the decode recurrence for 64 of the 4096 heads over
    the prefill and all steps, scaled to every head."""
    from threadpoolctl import threadpool_info

    from oracle import kata_oracle as orc

    blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    affinity = len(os.sched_getaffinity(0))
    t = time.perf_counter()
    orc.forward_chunked(inp.q64, inp.k64, inp.v64, w.chunk, w.eps)
    dt_chunked = time.perf_counter() - t
    t = time.perf_counter()
    orc.forward_quadratic(inp.q64[0, 0], inp.k64[0, 0], inp.v64[0, 0], w.eps)
    dt_quad = time.perf_counter() - t
    per_config = {w.name: {
        "chunked_s": round(dt_chunked, 2), "chunked_tokens_per_s": round(w.B * w.T / dt_chunked, 1),
        "quadratic_s_extrapolated": round(dt_quad * w.B * w.H, 1),
        "quadratic_tokens_per_s": round(w.B * w.T / (dt_quad * w.B * w.H), 1),
        "quadratic_sample": f"head (0,0), all {w.T} tokens ({dt_quad:.1f} s), times {w.B * w.H} heads"}}
    for cw in (ki.TINY, ki.MEDIUM, ki.WIDE):
        ci = ki.workload_inputs(cw)
        t = time.perf_counter()
        orc.forward_quadratic(ci.q64, ci.k64, ci.v64, cw.eps)
        dt = time.perf_counter() - t
        per_config[cw.name] = {"quadratic_s": round(dt, 3), "quadratic_tokens_per_s": round(cw.B * cw.T / dt, 1)}
    dw = ki.DECODE
    nh = 64
    di = ki.decode_inputs(dw.seed, nh, dw.prefill, dw.steps, dw.d, dw.dv)
    t = time.perf_counter()
    S, z = orc.decode_state(di.pk.astype(np.float64), di.pv.astype(np.float64))
    for s_ in range(dw.steps):
        S, z, _ = orc.decode_step(S, z, di.sq[s_], di.sk[s_], di.sv[s_], dw.eps)
    dt = (time.perf_counter() - t) * dw.heads / nh
    per_config[dw.name] = {"s_extrapolated": round(dt, 1), "tokens_per_s": round(dw.seqs * dw.steps / dt, 1),
                           "sample": f"{nh} of {dw.heads} heads (prefill and {dw.steps} steps), scaled"}
    return {"value": round(w.B * w.T / dt_chunked, 1), "unit": "tokens/s", "cores": min(blas, affinity),
            "kind": "oracle",
            "sample": f"fp64 chunked oracle (Eqs. 17-20) over the whole workload: {w.B * w.H} heads x "
                      f"{w.T} tokens in {dt_chunked:.1f} s; no extrapolation",
            "sample_seconds": round(dt_chunked, 2),
            "blas_threads": blas, "host_cpus": os.cpu_count(), "affinity_cpus": affinity,
            "per_config": per_config}


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch

    import associative_memory_amd as am
    import kata_inputs as ki

    am.lib()  # fails loudly when libkata.so is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    hip = Hip()

    if args.calib_copy:
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": 5}))
        return
    if args.calib_read:
        # reads 256 MiB once per launch and writes a few bytes
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        for _ in range(5):
            src.sum()
        torch.cuda.synchronize()
        print(json.dumps({"calib_read_bytes": n, "launches": 5}))
        return

    def progress(what):
        print(f"bench: {what}", file=sys.stderr, flush=True)

    progress("forward T=131072")
    w, inp, fwd = bench_forward(args, hip, am, ki, torch)
    main_r = fwd["auto"]
    D = w.d * (w.d + 1) // 2
    BHT = w.B * w.H * w.T
    flop_per_tok = 2 * ((w.chunk + 1) / 2 * (w.d + w.dv) + 2 * D * w.dv + 2 * D)
    bytes_per_tok = 2 * (2 * w.d + w.dv) + 2 * w.dv
    readout_ms = main_r["stage_ms"]["readout"]
    achieved = bytes_per_tok * BHT / (readout_ms * 1e-3) / 1e9
    rec = {
        "metric": "tokens/s + % bf16 MFMA peak, KATA chunked fwd T=131072; decode % HBM BW",
        "value": round(main_r["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_ms": args.warmup_ms,
        "ms_per_step": round(main_r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded unit-norm Gaussian q,k; Gaussian v)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d": w.d, "dv": w.dv,
                   "chunk": w.chunk, "plan": main_r["plan"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for("forward_readout"), "kernel": "readout",
                     "algorithmic_bytes_per_launch": bytes_per_tok * BHT},
        "mfma": {"useful_tflops": round(flop_per_tok * BHT / (main_r["ms_per_step"] * 1e-3) / 1e12, 2),
                 "peak_tflops": BF16_PEAK_TFLOPS,
                 "frac": round(flop_per_tok * BHT / (main_r["ms_per_step"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 5)},
        "head_tokens_per_s": round(BHT / (main_r["ms_per_step"] * 1e-3), 1),
        # max(time at HBM peak on the minimal bytes, time at bf16 MFMA peak on
        # the useful FLOPs) over the measured step: the fraction of the
        # attainable roofline the whole step reaches
        "attainable": {
            "t_hbm_us": round(bytes_per_tok * BHT / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
            "t_mfma_us": round(flop_per_tok * BHT / (BF16_PEAK_TFLOPS * 1e12) * 1e6, 2),
            "t_step_us": round(main_r["ms_per_step"] * 1e3, 2),
            "frac": round(max(bytes_per_tok * BHT / (HBM_PEAK_GBS * 1e9),
                              flop_per_tok * BHT / (BF16_PEAK_TFLOPS * 1e12))
                          / (main_r["ms_per_step"] * 1e-3), 4)},
        "timing": f"after an untimed warm-up of at least {args.warmup} forwards per variant and "
                  f"{args.warmup_ms:g} ms, median over {args.repeats} regions of exactly {args.steps} "
                  "forwards each, the three "
                  "prefix variants interleaved (rotating order), HIP events on the library's stream; "
                  "other_workloads the same way, each workload's plans interleaved",
        "scan_variants": {s: {"tokens_per_s": round(fwd[s]["tokens_per_s"], 1),
                              "ms_per_step": round(fwd[s]["ms_per_step"], 4),
                              "ms_per_step_samples": fwd[s]["ms_per_step_samples"],
                              "stage_ms": {kk: round(vv, 4) for kk, vv in fwd[s]["stage_ms"].items()},
                              "plan": fwd[s]["plan"]}
                          for s in ("sequential", "associative")},
    }
    progress("measured peaks")
    peaks = measure_peaks(hip, am, torch)
    peaks["readout_frac_of_copy_bw"] = round(achieved / peaks["hbm_copy_gbs"], 4)
    peaks["step_useful_frac_of_measured_mfma"] = round(
        flop_per_tok * BHT / (main_r["ms_per_step"] * 1e-3) / 1e12 / peaks["mfma_bf16_tflops"], 5)
    rec["measured_peaks"] = peaks
    if not args.no_other:
        progress("other forward workloads")
        rec["other_workloads"] = bench_other_workloads(args, hip, am, ki, torch)
    if not args.no_table8:
        progress("quadratic and chunked block maps, d = 64")
        rec["quadratic_block_maps_d64"] = bench_table8(args, hip, am, ki, torch)
    if not args.no_linear:
        progress("linear features")
        rec["linear_features_d64"] = bench_linear(args, hip, am, ki, torch)
    if not args.no_gated:
        progress("gated read")
        rec["gated"] = bench_gated(args, hip, am, ki, torch)
    progress("feature map")
    rec["feature_map"] = bench_feature_map(args, hip, am, ki, torch)
    if not args.no_decode:
        progress("decode")
        rec["decode"] = bench_decode(args, hip, am, ki, torch, ki.DECODE)
        rec["decode_beyond_cache"] = bench_decode(args, hip, am, ki, torch, ki.DECODE_512)
    if not args.no_cpu_baseline:
        progress("CPU oracle baseline")
        rec["cpu_baseline"] = cpu_baseline(w, inp, ki)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec))


if __name__ == "__main__":
    main()

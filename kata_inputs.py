"""Seeded synthetic inputs for the KATA rank-one-PSD linear-attention path.

This module is shared by the tests, the benchmark and the smoke check. It only
draws random numbers, normalises rows, rounds to the storage dtype and
describes the workload shapes. None of the method's arithmetic (feature map,
scores, states, readout) lives here, so both the fp64 oracle and the HIP path
can consume its outputs without sharing any computation.

Input recipe (the KATA page, "Kernelized Linear Attention: Breaking the
Capacity Wall with Symmetric Cones", Sec. 3 and App. E; the workloads below
follow the configuration list this library is measured on):
  * q, k rows are i.i.d. N(0, I_d) draws normalised to the unit sphere, v rows
    are i.i.d. N(0, I_dv);
  * draw order is q, then k, then v, each as a full C-order [B, H, T, .] fp64
    array from numpy's PCG64 generator with the workload's seed;
  * bf16 workloads round fp64 -> fp32 -> bf16, each step round-to-nearest-even;
    the oracle consumes exactly the rounded values the device receives.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class ForwardWorkload:
    name: str
    B: int
    H: int
    T: int
    d: int
    dv: int
    chunk: int
    dtype: str
    seed: int
    eps: float = 1e-6
    g: int = 1  # feature blocks of the KATA-Mg maps (1: the full map)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    seqs: int
    H: int
    d: int
    dv: int
    prefill: int
    steps: int
    dtype: str
    seed: int
    eps: float = 1e-6

    @property
    def heads(self) -> int:
        return self.seqs * self.H


# The five measured workloads: a tiny fp32 case, three bf16 forwards and the
# recurrent decode.
TINY = ForwardWorkload("tiny_T256_d16_dv16_C32_f32", 1, 1, 256, 16, 16, 32, F32, 0)
MEDIUM = ForwardWorkload("B4_H8_T2048_d16_dv64_C64_bf16", 4, 8, 2048, 16, 64, 64, BF16, 1)
WIDE = ForwardWorkload("B2_H16_T8192_d32_dv64_C64_bf16", 2, 16, 8192, 32, 64, 64, BF16, 2)
LONG = ForwardWorkload("B1_H8_T131072_d16_dv64_C128_bf16", 1, 8, 131072, 16, 64, 128, BF16, 3)
DECODE = DecodeWorkload("decode_256seq_H16_d16_dv64_prefill4096_1024steps_f32",
                        256, 16, 16, 64, 4096, 1024, F32, 4)
# the same decode with twice the sequences: 290 MB of state, more than the
# 256 MB Infinity Cache holds, so each step streams the state from HBM
DECODE_512 = DecodeWorkload("decode_512seq_H16_d16_dv64_prefill4096_1024steps_f32",
                            512, 16, 16, 64, 4096, 1024, F32, 5)

FORWARD_WORKLOADS = (TINY, MEDIUM, WIDE, LONG)


def table8(T: int, g: int, seed: int) -> ForwardWorkload:
    """The KATA page's forward-latency shape (Table 8: B = 8, H = 16,
    d_head = 64, bf16; dv = d_head) with the KATA-Mg map of g blocks."""
    return ForwardWorkload(f"B8_H16_T{T}_d64_dv64_M{g}_bf16", 8, 16, T, 64, 64, 64, BF16, seed, g=g)


# quadratic-form measurements on that shape: M1, M2, M4 at 1K, 4K and 16K tokens
TABLE8_QUAD = tuple(table8(T, g, 6 + 3 * i + j)
                    for i, T in enumerate((1024, 4096, 16384)) for j, g in enumerate((1, 2, 4)))


# ---------------------------------------------------------------- rounding

def round_f32(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32, round-to-nearest-even (IEEE default)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64/fp32 -> bf16 bit patterns (uint16), via fp32, round-to-nearest-even.

    Finite inputs only (the generators never produce NaN/Inf).
    """
    f = round_f32(x)
    u = f.view(np.uint32)
    # finite values stay below 0xFF800000, so the sum cannot wrap in 32 bits
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return u.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values."""
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def as_storage(x: np.ndarray, dtype: str):
    """Return (device_payload, exact_fp64_values) for storage dtype `dtype`.

    device_payload is float32 for F32 and uint16 bf16 bit patterns for BF16;
    exact_fp64_values is what those stored numbers equal, for the oracle.
    """
    if dtype == F32:
        f = round_f32(x)
        return f, f.astype(np.float64)
    if dtype == BF16:
        b = bf16_bits(x)
        return b, bf16_to_f64(b)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------- drawing

def unit_rows(g: np.random.Generator, shape) -> np.ndarray:
    x = g.standard_normal(shape)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


def draw_qkv(B: int, H: int, T: int, d: int, dv: int, seed: int):
    """fp64 q, k (unit rows) and v (Gaussian), drawn q -> k -> v."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = unit_rows(g, (B, H, T, d))
    k = unit_rows(g, (B, H, T, d))
    v = g.standard_normal((B, H, T, dv))
    return q, k, v


@dataclasses.dataclass
class ForwardInputs:
    """Device payloads (float32 or bf16 bits) and their exact fp64 values."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q64: np.ndarray
    k64: np.ndarray
    v64: np.ndarray
    dtype: str


def forward_inputs(B: int, H: int, T: int, d: int, dv: int, dtype: str, seed: int) -> ForwardInputs:
    q, k, v = draw_qkv(B, H, T, d, dv, seed)
    qs, q64 = as_storage(q, dtype)
    ks, k64 = as_storage(k, dtype)
    vs, v64 = as_storage(v, dtype)
    return ForwardInputs(qs, ks, vs, q64, k64, v64, dtype)


def workload_inputs(w: ForwardWorkload) -> ForwardInputs:
    return forward_inputs(w.B, w.H, w.T, w.d, w.dv, w.dtype, w.seed)


@dataclasses.dataclass
class DecodeInputs:
    """Per-head history (prefill) tokens and the per-step tokens.

    Shapes: pk [heads, P, d], pv [heads, P, dv]; sq, sk [steps, heads, d],
    sv [steps, heads, dv]. All float32 (the decode workload is fp32), with the
    fp64 values equal to them.
    """
    pk: np.ndarray
    pv: np.ndarray
    sq: np.ndarray
    sk: np.ndarray
    sv: np.ndarray


def decode_head_inputs(seed: int, head: int, prefill: int, steps: int, d: int, dv: int):
    """One head's history and step tokens from its own stream, so any subset
    of heads can be regenerated alone.  Returns float32 arrays
    (pk [P,d], pv [P,dv], sq [S,d], sk [S,d], sv [S,dv])."""
    g = np.random.Generator(np.random.PCG64([seed, head]))
    pk = unit_rows(g, (prefill, d))
    pv = g.standard_normal((prefill, dv))
    sq = unit_rows(g, (steps, d))
    sk = unit_rows(g, (steps, d))
    sv = g.standard_normal((steps, dv))
    return tuple(round_f32(a) for a in (pk, pv, sq, sk, sv))


def decode_inputs(seed: int, heads: int, prefill: int, steps: int, d: int, dv: int,
                  head_ids: Optional[np.ndarray] = None) -> DecodeInputs:
    ids = np.arange(heads) if head_ids is None else np.asarray(head_ids)
    per = [decode_head_inputs(seed, int(h), prefill, steps, d, dv) for h in ids]
    pk = np.stack([p[0] for p in per])
    pv = np.stack([p[1] for p in per])
    sq = np.stack([p[2] for p in per], axis=1)
    sk = np.stack([p[3] for p in per], axis=1)
    sv = np.stack([p[4] for p in per], axis=1)
    return DecodeInputs(pk, pv, sq, sk, sv)


def decode_inputs_torch(seed: int, heads: int, prefill: int, steps: int, d: int, dv: int,
                        device):
    """Full-size decode inputs drawn on the device with torch's seeded
    generator (the host draw of ~1.7e9 normals would take minutes).  Same
    distributions as decode_inputs; returns float32 tensors
    (pk [heads,P,d], pv [heads,P,dv], sq [S,heads,d], sk [S,heads,d],
    sv [S,heads,dv])."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def unit(shape):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)

    pk = unit((heads, prefill, d))
    pv = torch.randn((heads, prefill, dv), generator=gen, device=device, dtype=torch.float32)
    sq = unit((steps, heads, d))
    sk = unit((steps, heads, d))
    sv = torch.randn((steps, heads, dv), generator=gen, device=device, dtype=torch.float32)
    return pk, pv, sq, sk, sv


def forward_inputs_torch(B: int, H: int, T: int, d: int, dv: int, seed: int, device):
    """bf16 q, k (unit rows) and v (Gaussian) drawn on the device with
    torch's seeded generator, for timing large shapes (same distributions as
    forward_inputs, not the same numbers)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def unit(shape):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return (x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)).to(torch.bfloat16)

    q = unit((B, H, T, d))
    k = unit((B, H, T, d))
    v = torch.randn((B, H, T, dv), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v


def draw_log_gamma(B: int, H: int, T: int, seed: int) -> np.ndarray:
    """Per-token log gates for the gated read, float32 [B, H, T]:
    log gamma = log sigmoid(u) with u ~ N(4, 1) i.i.d. (gates mostly 0.95 to
    0.995, a memory of tens to hundreds of tokens), from PCG64([seed, 1])."""
    g = np.random.Generator(np.random.PCG64([seed, 1]))
    u = g.standard_normal((B, H, T)) + 4.0
    return round_f32(-np.log1p(np.exp(-u)))

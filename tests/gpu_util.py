"""Helpers for the GPU parity tests: move seeded inputs to the device, pull
results back, and apply the parity bar.

Parity bar (max abs error against the fp64 oracle on the same inputs):
  fp32 inputs:  <= 1e-4 * max|v|
  bf16 inputs:  <= 2e-2 * max|v|   (bf16 operands, fp32 accumulation)
At long T the outputs shrink like 1/sqrt(T) while max|v| does not, so the
bar alone stops meaning much; every check therefore also bounds the
root-mean-square error relative to the root-mean-square reference output
(1e-5 for fp32, 1e-2 for bf16), which a wrong state or a dropped term fails.
"""
import sys

import numpy as np
import torch

import kata_inputs as ki

DEV = "cuda"

ABS_TOL = {ki.F32: 1e-4, ki.BF16: 2e-2}
RMS_TOL = {ki.F32: 1e-5, ki.BF16: 1e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(payload: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(payload)
    if dtype == ki.BF16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(got: np.ndarray, ref: np.ndarray, dtype: str, vmax: float, what: str = ""):
    """Assert the parity bar; returns (max_abs_err, rms_rel_err)."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    rms_ref = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    rms_rel = float(np.sqrt(np.mean(err * err)) / rms_ref) if rms_ref > 0 else 0.0
    say(f"  {what}: max_abs_err={mx:.3e} (bar {ABS_TOL[dtype] * vmax:.3e}) "
        f"rms_rel={rms_rel:.3e} (bar {RMS_TOL[dtype]:.1e})")
    assert mx <= ABS_TOL[dtype] * vmax, f"{what}: max abs err {mx} > {ABS_TOL[dtype]} * {vmax}"
    assert rms_rel <= RMS_TOL[dtype], f"{what}: rms rel err {rms_rel} > {RMS_TOL[dtype]}"
    return mx, rms_rel


# ------------------------------------------------------------------ guard bands
#
# An output (or state) tensor placed inside a larger buffer whose margins hold
# a fill pattern: any write past either end of the tensor changes the pattern.
GUARD = 4096  # elements on each side


def _fill_bits(dtype):
    # bf16 0x7FA5 and fp32 0x7FA5A5A5 are quiet NaNs no kernel writes
    return 0x7FA5 if dtype == torch.bfloat16 else 0x7FA5A5A5


def guarded(shape, dtype):
    """(buffer, view): `view` of `shape` inside `buffer` with GUARD canary
    elements on both sides."""
    n = int(np.prod(shape))
    if dtype == torch.bfloat16:
        buf = torch.full((n + 2 * GUARD,), _fill_bits(dtype), dtype=torch.int16, device=DEV)
        view = buf[GUARD:GUARD + n].view(torch.bfloat16).view(shape)
    else:
        buf = torch.full((n + 2 * GUARD,), _fill_bits(dtype), dtype=torch.int32, device=DEV)
        view = buf[GUARD:GUARD + n].view(torch.float32).view(shape)
    return buf, view


def assert_guards(buf, what=""):
    fill = int(buf[0].item())
    head, tail = buf[:GUARD], buf[-GUARD:]
    assert torch.all(head == fill) and torch.all(tail == fill), f"{what}: write outside the tensor"


def guarded_workspace(need):
    """(buffer, workspace view of `need` bytes, guard bytes after it)."""
    buf = torch.full((need + GUARD,), 0x5A, dtype=torch.uint8, device=DEV)
    return buf, buf[:max(need, 1)]


def assert_workspace_guard(buf, need, what=""):
    assert torch.all(buf[need:] == 0x5A), f"{what}: write past the workspace"

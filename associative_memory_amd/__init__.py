"""Python binding of libkata (causal linear attention with KATA's rank-one PSD
feature map on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libkata.so.  PyTorch supplies device memory and the current stream.
The Python functions carry the C entry points' names (include/kata.h) and take
tensors instead of raw pointers and sizes.  The library must have been built
(`python -m associative_memory_amd.build`); importing the functions without it
raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
# KATA_LIBRARY names another build of the same library (e.g. one whose host
# code carries the address and undefined-behaviour sanitizers).
LIB_PATH = os.environ.get("KATA_LIBRARY") or os.path.join(_HERE, "libkata.so")

KATA_F32 = 0
KATA_BF16 = 1
KATA_SCAN_AUTO = 0
KATA_SCAN_SEQUENTIAL = 1
KATA_SCAN_ASSOCIATIVE = 2
KATA_SCAN_RECOMPUTE = 3
KATA_SCAN_FUSED = 4
KATA_OK = 0

_SCANS = {"auto": KATA_SCAN_AUTO, "sequential": KATA_SCAN_SEQUENTIAL, "seq": KATA_SCAN_SEQUENTIAL,
          "associative": KATA_SCAN_ASSOCIATIVE, "assoc": KATA_SCAN_ASSOCIATIVE,
          "recompute": KATA_SCAN_RECOMPUTE, "fused": KATA_SCAN_FUSED}

EXPORTED = (
    "kata_status_string",
    "kata_feature_dim",
    "kata_feature_map",
    "kata_forward_workspace_bytes",
    "kata_forward_chunked",
    "kata_forward_chunked_noalloc",
    "kata_prefill_state",
    "kata_decode_step",
    "kata_forward_plan",
    "kata_forward_chunked_profiled",
    "kata_forward_quadratic",
    "kata_forward_linear_workspace_bytes",
    "kata_forward_linear",
    "kata_forward_gated_workspace_bytes",
    "kata_forward_gated",
    "kata_decode_step_gated",
    "kata_prefill_state_gated",
    "kata_forward_chunked_blocks_workspace_bytes",
    "kata_forward_chunked_blocks",
    "kata_probe_mfma_bf16",
)


class KataError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkata.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libkata.so not found at {LIB_PATH}; build it with "
                           "`python -m associative_memory_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.kata_status_string.restype = ctypes.c_char_p
    L.kata_status_string.argtypes = [i32]
    L.kata_feature_dim.restype = i64
    L.kata_feature_dim.argtypes = [i32]
    L.kata_feature_map.restype = i32
    L.kata_feature_map.argtypes = [vp, vp, i64, i32, i32, i32, vp]
    L.kata_forward_workspace_bytes.restype = sz
    L.kata_forward_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32, i32]
    L.kata_forward_chunked.restype = i32
    L.kata_forward_chunked.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, f32, i32, i32,
                                       vp, sz, vp]
    L.kata_forward_chunked_noalloc.restype = i32
    L.kata_forward_chunked_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, f32, i32, i32,
                                               vp]
    L.kata_prefill_state.restype = i32
    L.kata_prefill_state.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, vp]
    L.kata_decode_step.restype = i32
    L.kata_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp]
    L.kata_forward_chunked_profiled.restype = i32
    L.kata_forward_chunked_profiled.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, f32,
                                                i32, i32, vp, sz, vp, vp]
    L.kata_forward_quadratic.restype = i32
    L.kata_forward_quadratic.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, f32, i32, vp]
    L.kata_forward_linear_workspace_bytes.restype = sz
    L.kata_forward_linear_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32]
    L.kata_forward_linear.restype = i32
    L.kata_forward_linear.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, i32, f32, f32, i32,
                                      i32, vp, sz, vp]
    L.kata_forward_gated_workspace_bytes.restype = sz
    L.kata_forward_gated_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32]
    L.kata_forward_gated.restype = i32
    L.kata_forward_gated.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, i32, vp, sz, vp]
    L.kata_prefill_state_gated.restype = i32
    L.kata_prefill_state_gated.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, vp]
    L.kata_decode_step_gated.restype = i32
    L.kata_decode_step_gated.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    L.kata_forward_chunked_blocks_workspace_bytes.restype = sz
    L.kata_forward_chunked_blocks_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32]
    L.kata_forward_chunked_blocks.restype = i32
    L.kata_forward_chunked_blocks.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, i32, f32, i32,
                                              i32, vp, sz, vp]
    L.kata_forward_plan.restype = i32
    L.kata_forward_plan.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32, ctypes.c_char_p, sz]
    L.kata_probe_mfma_bf16.restype = i64
    L.kata_probe_mfma_bf16.argtypes = [vp, i32, i32, vp]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().kata_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != KATA_OK:
        raise KataError(status, where)


# ------------------------------------------------------------------ helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return KATA_F32
    if t.dtype == torch.bfloat16:
        return KATA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _scan_code(scan) -> int:
    if isinstance(scan, int):
        return scan
    return _SCANS[scan]


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> int:
    return t.data_ptr()


def _device_tensor(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ------------------------------------------------------------------ entry points

def kata_feature_dim(d: int) -> int:
    return int(lib().kata_feature_dim(int(d)))


def kata_feature_map(x, phi_dtype=None, out=None, stream=None):
    """phi(x) for x [..., d] -> [..., d(d+1)/2] (sqrt(2) off-diagonal packing)."""
    torch = _torch()
    _device_tensor(x, "x")
    d = x.shape[-1]
    D = kata_feature_dim(d)
    rows = x.numel() // d
    if out is None:
        out = torch.empty(x.shape[:-1] + (D,), dtype=phi_dtype or x.dtype, device=x.device)
    _device_tensor(out, "out")
    st = lib().kata_feature_map(_ptr(x), _ptr(out), rows, d, _dtype_code(x), _dtype_code(out),
                                _stream(stream))
    _check(st, "kata_feature_map")
    return out


def kata_forward_workspace_bytes(B, H, T, d, dv, chunk, scan="auto") -> int:
    return int(lib().kata_forward_workspace_bytes(B, H, T, d, dv, chunk, _scan_code(scan)))


def kata_probe_mfma_bf16(sink, workgroups: int, iters: int, stream=None) -> int:
    """Measurement aid: launch the matrix-core rate probe (see include/kata.h)
    on `stream`; sink is a float32 device tensor of >= workgroups * 256
    elements.  Returns the launch's FLOP count."""
    if sink.dtype != _torch().float32 or sink.numel() < workgroups * 256 or not sink.is_cuda:
        raise ValueError("sink: float32 device tensor of >= workgroups * 256 elements")
    flops = int(lib().kata_probe_mfma_bf16(sink.data_ptr(), workgroups, iters, _stream(stream)))
    if flops < 0:
        raise RuntimeError("kata_probe_mfma_bf16: invalid arguments or launch error")
    return flops


def kata_forward_plan(B, H, T, d, dv, chunk, dtype_code=KATA_BF16, scan="auto") -> str:
    buf = ctypes.create_string_buffer(512)
    st = lib().kata_forward_plan(B, H, T, d, dv, chunk, dtype_code, _scan_code(scan), buf, 512)
    _check(st, "kata_forward_plan")
    return buf.value.decode()


def kata_forward_chunked(q, k, v, chunk: int, eps: float = 1e-6, scan="auto", out=None,
                         workspace=None, stream=None):
    """Causal normalised read o_t = sum_{s<=t}(q_t.k_s)^2 v_s / (sum + eps).

    q, k: [B, H, T, d]; v: [B, H, T, dv]; float32 or bfloat16, contiguous,
    on the device.  scan: "auto", "sequential", "associative", "recompute"
    or "fused" (kata_scan_t).  Returns out [B, H, T, dv] (same dtype).
    """
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _device_tensor(t, n)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=v.dtype, device=v.device)
    _device_tensor(out, "out")
    sc = _scan_code(scan)
    need = kata_forward_workspace_bytes(B, H, T, d, dv, chunk, sc)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wptr = _ptr(workspace) if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().kata_forward_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, T, d, dv, chunk,
                                    float(eps), _dtype_code(q), sc, wptr, wbytes, _stream(stream))
    _check(st, "kata_forward_chunked")
    return out


KATA_NOALLOC_SCRATCH_BYTES = 64 << 20


def kata_forward_chunked_noalloc(q, k, v, chunk: int, eps: float = 1e-6, scan="auto", out=None,
                                 stream=None):
    """kata_forward_chunked with the library's static device scratch as its
    workspace: allocates nothing when `out` is given.  Shapes whose workspace
    exceeds KATA_NOALLOC_SCRATCH_BYTES raise (KATA_ERR_WORKSPACE); calls that
    overlap in time on one device race on the shared scratch."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _device_tensor(t, n)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=v.dtype, device=v.device)
    _device_tensor(out, "out")
    st = lib().kata_forward_chunked_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, T, d, dv, chunk,
                                            float(eps), _dtype_code(q), _scan_code(scan), _stream(stream))
    _check(st, "kata_forward_chunked_noalloc")
    return out


def kata_forward_quadratic(q, k, v, eps: float = 1e-6, g: int = 1, out=None, stream=None):
    """The causal read in its direct O(T^2) form (no state, no workspace),
    with the KATA-Mg score sum_a (q_a . k_a)^2 over g blocks of q and k
    (g = 1: the full map's (q . k)^2).  q, k: [B, H, T, d]; v: [B, H, T, dv];
    bf16, contiguous, on the device.  Returns out [B, H, T, dv] bf16."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _device_tensor(t, n)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=v.dtype, device=v.device)
    _device_tensor(out, "out")
    st = lib().kata_forward_quadratic(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, T, d, dv,
                                      int(g), float(eps), _dtype_code(q), _stream(stream))
    _check(st, "kata_forward_quadratic")
    return out


class StageEvents(ctypes.Structure):
    """kata_stage_events_t: hipEvent_t handles around the three forward stages."""
    _fields_ = [("stage_begin", ctypes.c_void_p * 3), ("stage_end", ctypes.c_void_p * 3)]


def kata_forward_chunked_profiled(q, k, v, chunk: int, events: "StageEvents", eps: float = 1e-6,
                                  scan="auto", out=None, workspace=None, stream=None):
    """kata_forward_chunked recording caller-owned hipEvent_t handles around
    each stage (span states, prefix, readout)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _device_tensor(t, n)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=v.dtype, device=v.device)
    sc = _scan_code(scan)
    need = kata_forward_workspace_bytes(B, H, T, d, dv, chunk, sc)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wptr = _ptr(workspace) if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().kata_forward_chunked_profiled(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, T, d, dv,
                                             chunk, float(eps), _dtype_code(q), sc, wptr, wbytes,
                                             ctypes.byref(events), _stream(stream))
    _check(st, "kata_forward_chunked_profiled")
    return out


def kata_prefill_state(k, v, S=None, z=None, stream=None) -> Tuple[object, object]:
    """Decode state of a history: S [B*H, D, dv] fp32, z [B*H, D] fp32."""
    torch = _torch()
    _device_tensor(k, "k")
    _device_tensor(v, "v")
    B, H, T, d = k.shape
    dv = v.shape[-1]
    D = kata_feature_dim(d)
    if S is None:
        S = torch.empty((B * H, D, dv), dtype=torch.float32, device=k.device)
    if z is None:
        z = torch.empty((B * H, D), dtype=torch.float32, device=k.device)
    st = lib().kata_prefill_state(_ptr(k), _ptr(v), _ptr(S), _ptr(z), B, H, T, d, dv,
                                  _dtype_code(k), _stream(stream))
    _check(st, "kata_prefill_state")
    return S, z


def kata_decode_step(S, z, q, k, v, eps: float = 1e-6, out=None, B: Optional[int] = None,
                     stream=None):
    """One recurrent step for every head: q, k [BH, d]; v [BH, dv]; S, z fp32
    state updated in place.  Returns out [BH, dv]."""
    torch = _torch()
    for t, n in ((S, "S"), (z, "z"), (q, "q"), (k, "k"), (v, "v")):
        _device_tensor(t, n)
    BH, d = q.shape[0], q.shape[-1]
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((BH, dv), dtype=v.dtype, device=v.device)
    b = 1 if B is None else B
    st = lib().kata_decode_step(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), b,
                                BH // b, d, dv, float(eps), _dtype_code(q), _stream(stream))
    _check(st, "kata_decode_step")
    return out


KATA_FEATURE_ORTHANT = 0
KATA_FEATURE_LORENTZ = 1
KATA_FEATURE_IDENTITY = 2
_FEATURES = {"orthant": KATA_FEATURE_ORTHANT, "lorentz": KATA_FEATURE_LORENTZ,
             "identity": KATA_FEATURE_IDENTITY}


def kata_forward_linear_workspace_bytes(B, H, T, d, dv, chunk=64) -> int:
    return int(lib().kata_forward_linear_workspace_bytes(B, H, T, d, dv, chunk))


def kata_forward_linear(q, k, v, feature: str = "orthant", shift: float = 1e-6, eps: float = 1e-6,
                        chunk: int = 64, scan="auto", out=None, workspace=None, stream=None):
    """Causal read with a linear feature: the orthant (ReLU(x) + shift) or
    Lorentz ((y, |y|(1 + s^2))) map read normalised,
    o_t = sum_{s<=t} (psi(q_t).psi(k_s)) v_s / (sum + eps), or the identity
    map read without a denominator, o_t = sum_{s<=t} (q_t.k_s) v_s.
    q, k: [B, H, T, d]; v: [B, H, T, dv]; bf16, contiguous, on the device.
    Returns out [B, H, T, dv] bf16."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _device_tensor(t, n)
    if feature not in _FEATURES:
        raise ValueError(f"feature must be one of {sorted(_FEATURES)}, got {feature!r}")
    B, H, T, d = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=v.dtype, device=v.device)
    _device_tensor(out, "out")
    need = kata_forward_linear_workspace_bytes(B, H, T, d, dv, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wptr = _ptr(workspace) if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().kata_forward_linear(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, T, d, dv, chunk,
                                   _FEATURES[feature], float(shift), float(eps), _dtype_code(q),
                                   _scan_code(scan), wptr, wbytes, _stream(stream))
    _check(st, "kata_forward_linear")
    return out


def kata_forward_gated_workspace_bytes(B, H, T, d, dv, chunk=128) -> int:
    return int(lib().kata_forward_gated_workspace_bytes(B, H, T, d, dv, chunk))


def kata_forward_gated(q, k, v, log_gamma, chunk: int = 128, out=None, workspace=None, stream=None):
    """GatedKATA read o_t = phi(q_t)^T S_t with S_t = gamma_t S_{t-1} +
    phi(k_t) v_t^T (no denominator).  q, k: [B, H, T, d]; v: [B, H, T, dv];
    bf16; log_gamma: [B, H, T] float32; all contiguous on the device.
    Returns out [B, H, T, dv] bf16."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (log_gamma, "log_gamma")):
        _device_tensor(t, n)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    if tuple(log_gamma.shape) != (B, H, T) or log_gamma.dtype != torch.float32:
        raise ValueError("log_gamma must be a float32 tensor of shape [B, H, T]")
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=v.dtype, device=v.device)
    _device_tensor(out, "out")
    need = kata_forward_gated_workspace_bytes(B, H, T, d, dv, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wptr = _ptr(workspace) if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().kata_forward_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma), _ptr(out), B, H, T, d, dv,
                                  chunk, _dtype_code(q), wptr, wbytes, _stream(stream))
    _check(st, "kata_forward_gated")
    return out


def kata_prefill_state_gated(k, v, log_gamma, S=None, stream=None):
    """GatedKATA state of a history (S_t = gamma_t S_{t-1} + phi(k_t) v_t^T):
    k [B, H, T, d], v [B, H, T, dv], log_gamma [B, H, T] float32, all on the
    device.  Returns S [B*H, D, dv] float32, the layout kata_decode_step_gated
    continues from."""
    torch = _torch()
    for t, n in ((k, "k"), (v, "v"), (log_gamma, "log_gamma")):
        _device_tensor(t, n)
    B, H, T, d = k.shape
    dv = v.shape[-1]
    if tuple(log_gamma.shape) != (B, H, T) or log_gamma.dtype != torch.float32:
        raise ValueError("log_gamma must be a float32 tensor of shape [B, H, T]")
    D = kata_feature_dim(d)
    if S is None:
        S = torch.empty((B * H, D, dv), dtype=torch.float32, device=k.device)
    _device_tensor(S, "S")
    st = lib().kata_prefill_state_gated(_ptr(k), _ptr(v), _ptr(log_gamma), _ptr(S), B, H, T, d, dv,
                                        _dtype_code(k), _stream(stream))
    _check(st, "kata_prefill_state_gated")
    return S


def kata_decode_step_gated(S, q, k, v, log_gamma, out=None, stream=None):
    """One GatedKATA step in place: S = exp(log_gamma) S + phi(k) v^T, then
    out = phi(q)^T S.  S: [BH, D, dv] float32; q, k: [BH, d]; v: [BH, dv];
    log_gamma: [BH] float32.  Returns out [BH, dv] (dtype of v)."""
    torch = _torch()
    for t, n in ((S, "S"), (q, "q"), (k, "k"), (v, "v"), (log_gamma, "log_gamma")):
        _device_tensor(t, n)
    BH, d = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((BH, dv), dtype=v.dtype, device=v.device)
    _device_tensor(out, "out")
    st = lib().kata_decode_step_gated(_ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma), _ptr(out),
                                      1, BH, d, dv, _dtype_code(q), _stream(stream))
    _check(st, "kata_decode_step_gated")
    return out


def kata_forward_chunked_blocks(q, k, v, g: int, chunk: int = 64, eps: float = 1e-6, scan="auto",
                                out=None, workspace=None, stream=None):
    """The chunked read with the KATA-Mg score sum_a (q_a . k_a)^2 over g
    blocks (g = 1: kata_forward_chunked).  q, k: [B, H, T, d]; v: [B, H, T, dv];
    contiguous on the device.  Returns out [B, H, T, dv]."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _device_tensor(t, n)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=v.dtype, device=v.device)
    _device_tensor(out, "out")
    sc = _scan_code(scan)
    need = int(lib().kata_forward_chunked_blocks_workspace_bytes(B, H, T, d, dv, g, chunk, sc))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wptr = _ptr(workspace) if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().kata_forward_chunked_blocks(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, T, d, dv, g, chunk,
                                           float(eps), _dtype_code(q), sc, wptr, wbytes, _stream(stream))
    _check(st, "kata_forward_chunked_blocks")
    return out

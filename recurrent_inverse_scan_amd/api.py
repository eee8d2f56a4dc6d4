"""Python front end of the VLA scan library (argument marshalling only).

Torch provides device memory and the current HIP stream; every step of the
scan and of the projection runs in the HIP kernels of libvla.so, called
through the C ABI (``_lib``).
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib

_DT = {torch.float32: _lib.VLA_F32, torch.bfloat16: _lib.VLA_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("VLA tensors must live on a HIP device")


def _seq_strides(q, k, v):
    """(stride_b, stride_h, stride_t) for the ABI: zeros when q, k, v are
    contiguous, else their shared element strides (feature dimension
    contiguous)."""
    if all(t.is_contiguous() for t in (q, k, v)):
        return (0, 0, 0)
    if not (q.stride() == k.stride() == v.stride()) or q.stride(-1) != 1:
        raise ValueError("strided q, k, v must share their strides and keep the feature dimension contiguous")
    return tuple(int(x) for x in q.stride()[:3])


def _check_out(t, shape, dtype, dev, name):
    if (tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != dev or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {dev} "
                         f"(got {t.dtype} {tuple(t.shape)} on {t.device}, contiguous={t.is_contiguous()})")


def make_params(B, H, T, d, r, dtype, *, eps=1e-6, nudge_period=0, s_cap=None, den_eps=1e-6, t0=0,
                schedule="auto", validate=False, chunk_len=0, segment_blocks=0,
                update="additive", strides=(0, 0, 0), para_segments=0) -> _lib.ScanParams:
    p = _lib.ScanParams()
    _lib.load().vla_scan_params_init(ctypes.byref(p))
    p.B, p.H, p.T, p.d, p.r = B, H, T, d, r
    p.in_dtype = _DT[dtype]
    p.eps = eps
    p.nudge_period = nudge_period
    p.s_cap = 0.0 if (s_cap is None or not math.isfinite(s_cap) or s_cap <= 0) else float(s_cap)
    p.den_eps = den_eps
    p.t0 = t0
    p.stride_b, p.stride_h, p.stride_t = strides
    p.schedule = {"auto": _lib.VLA_SCHEDULE_AUTO, "sequential": _lib.VLA_SCHEDULE_SEQUENTIAL,
                  "chunked": _lib.VLA_SCHEDULE_CHUNKED}[schedule]
    p.validate = 1 if validate else 0
    p.chunk_len = chunk_len
    p.segment_blocks = segment_blocks
    p.update = {"additive": _lib.VLA_UPDATE_ADDITIVE, "residual": _lib.VLA_UPDATE_RESIDUAL}[update]
    p.para_segments = para_segments
    return p


def scan_forward(q, k, v, u, A0=None, S0=None, n0=None, *, eps=1e-6, nudge_period=0, s_cap=None,
                 den_eps=1e-6, t0=0, schedule="auto", validate=False, chunk_len=0, segment_blocks=0, out=None,
                 workspace=None, update="additive", para_segments=0):
    """Run vla_scan_forward.

    q, k, v: [B, H, T, d]; u: [B, H, T, r, d], all float32 or all bfloat16 on
    the device.  q, k, v may be strided views (e.g. slices of one packed
    projection) if they share their strides and keep the feature dimension
    contiguous; the library gathers them into its workspace.  A0, S0
    [B, H, d, d] and n0 [B, H, d] are float32 or None.
    ``schedule`` is "auto", "sequential" or "chunked"; ``chunk_len`` 0 lets
    the library pick; ``segment_blocks`` (chunked schedule) sets the blocks of
    64 tokens per state-pass segment, 0 lets the library pick and -1 keeps one
    segment.  ``para_segments`` (chunked schedule, additive update) cuts each
    chain's state pass into that many segments iterated in parallel (2..16),
    1 keeps one pass per chain, 0 lets the library pick.  ``update`` is
    "additive" or "residual" (the delta-rule state step; both schedules).  ``out`` may pass preallocated (o, A_T, S_T, n_T,
    stats) tensors and ``workspace`` a preallocated uint8 device buffer of at
    least ``workspace_size(...)`` bytes.  Returns (o, A_T, S_T, n_T, stats).
    """
    if q.dim() != 4 or u.dim() != 5:
        raise ValueError("q, k, v must be [B, H, T, d] and u [B, H, T, r, d]")
    B, H, T, d = q.shape
    r = u.shape[3]
    dt = q.dtype
    if dt not in _DT or any(x.dtype != dt for x in (k, v, u)):
        raise ValueError("q, k, v, u must share one dtype: float32 or bfloat16")
    if k.shape != q.shape or v.shape != q.shape or tuple(u.shape) != (B, H, T, r, d):
        raise ValueError("shape mismatch among q, k, v, u")
    if not u.is_contiguous():
        raise ValueError("u must be contiguous")
    strides = _seq_strides(q, k, v)
    dev = q.device
    if any(t is not None and t.device != dev for t in (k, v, u, A0, S0, n0)):
        raise ValueError("every tensor must be on the device of q")
    for t, shp in ((A0, (B, H, d, d)), (S0, (B, H, d, d)), (n0, (B, H, d))):
        if t is not None and (tuple(t.shape) != shp or t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("A0/S0/n0 must be contiguous float32 of shape [B,H,d,d]/[B,H,d,d]/[B,H,d]")
    if out is None:
        o = torch.empty((B, H, T, d), device=dev, dtype=dt)
        A_T = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
        S_T = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
        n_T = torch.empty((B, H, d), device=dev, dtype=torch.float32)
        stats = torch.empty((B, H, 4), device=dev, dtype=torch.int32)
    else:
        o, A_T, S_T, n_T, stats = out
        _check_out(o, (B, H, T, d), dt, dev, "o")
        _check_out(A_T, (B, H, d, d), torch.float32, dev, "A_T")
        _check_out(S_T, (B, H, d, d), torch.float32, dev, "S_T")
        _check_out(n_T, (B, H, d), torch.float32, dev, "n_T")
        if stats is not None:
            _check_out(stats, (B, H, 4), torch.int32, dev, "stats")
    if workspace is not None and (workspace.dtype != torch.uint8 or workspace.device != dev
                                  or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {dev}")
    _need_cuda(q, k, v, u, A0, S0, n0, o, A_T, S_T, n_T, stats, workspace)
    p = make_params(B, H, T, d, r, dt, eps=eps, nudge_period=nudge_period, s_cap=s_cap, den_eps=den_eps,
                    t0=t0, schedule=schedule, validate=validate, chunk_len=chunk_len,
                    segment_blocks=segment_blocks, update=update, strides=strides, para_segments=para_segments)
    lib = _lib.load()
    ws_bytes = ctypes.c_size_t(0)
    _lib.check(lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(ws_bytes)))
    ws = workspace
    if ws_bytes.value and (ws is None or ws.numel() < ws_bytes.value):
        ws = torch.empty(ws_bytes.value, device=dev, dtype=torch.uint8)
    with torch.cuda.device(dev):
        _lib.check(lib.vla_scan_forward(
            ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(A0), _ptr(S0), _ptr(n0),
            _ptr(o), _ptr(A_T), _ptr(S_T), _ptr(n_T), _ptr(stats), _ptr(ws) if ws_bytes.value else None,
            ws_bytes.value,
            _stream_ptr(dev)))
    return o, A_T, S_T, n_T, stats


def scan_forward_noalloc(q, k, v, u, A0=None, S0=None, n0=None, *, out, eps=1e-6, nudge_period=0, s_cap=None,
                         den_eps=1e-6, t0=0, schedule="auto", validate=False, chunk_len=0, segment_blocks=0,
                         update="additive"):
    """Run vla_scan_forward_noalloc: scan_forward with the library's static
    per-device scratch instead of a workspace.  ``out`` = (o, A_T, S_T, n_T,
    stats) must be preallocated (stats may be None); nothing is allocated.
    Calls that overlap on one device race on the shared scratch."""
    if q.dim() != 4 or u.dim() != 5:
        raise ValueError("q, k, v must be [B, H, T, d] and u [B, H, T, r, d]")
    B, H, T, d = q.shape
    r = u.shape[3]
    dt = q.dtype
    if dt not in _DT or any(x.dtype != dt for x in (k, v, u)):
        raise ValueError("q, k, v, u must share one dtype: float32 or bfloat16")
    if k.shape != q.shape or v.shape != q.shape or tuple(u.shape) != (B, H, T, r, d) or not u.is_contiguous():
        raise ValueError("shape mismatch among q, k, v, u (u contiguous)")
    dev = q.device
    for t, shp in ((A0, (B, H, d, d)), (S0, (B, H, d, d)), (n0, (B, H, d))):
        if t is not None:
            _check_out(t, shp, torch.float32, dev, "A0/S0/n0")
    o, A_T, S_T, n_T, stats = out
    _check_out(o, (B, H, T, d), dt, dev, "o")
    _check_out(A_T, (B, H, d, d), torch.float32, dev, "A_T")
    _check_out(S_T, (B, H, d, d), torch.float32, dev, "S_T")
    _check_out(n_T, (B, H, d), torch.float32, dev, "n_T")
    if stats is not None:
        _check_out(stats, (B, H, 4), torch.int32, dev, "stats")
    strides = _seq_strides(q, k, v)
    _need_cuda(q, k, v, u, A0, S0, n0, o, A_T, S_T, n_T, stats)
    p = make_params(B, H, T, d, r, dt, eps=eps, nudge_period=nudge_period, s_cap=s_cap, den_eps=den_eps,
                    t0=t0, schedule=schedule, validate=validate, chunk_len=chunk_len,
                    segment_blocks=segment_blocks, update=update, strides=strides)
    lib = _lib.load()
    with torch.cuda.device(dev):
        _lib.check(lib.vla_scan_forward_noalloc(
            ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(A0), _ptr(S0), _ptr(n0),
            _ptr(o), _ptr(A_T), _ptr(S_T), _ptr(n_T), _ptr(stats), _stream_ptr(dev)))
    return o, A_T, S_T, n_T, stats


def scan_forward_fused(q_raw, k_raw, v, W_u, A0=None, S0=None, n0=None, *, eps=1e-6, nudge_period=0, s_cap=None,
                       den_eps=1e-6, t0=0, schedule="auto", chunk_len=0, segment_blocks=0, update="additive",
                       out=None, workspace=None):
    """Run vla_scan_forward_fused: the scan from the raw inputs, with
    q, k = ELU(.) + 1 and u = normalize(W_u[i] k_raw) computed by the library.

    q_raw, k_raw, v: [B, H, T, d]; W_u: [r, d, d]; one dtype (float32 or
    bfloat16), contiguous.  Other arguments and the result as scan_forward."""
    if q_raw.dim() != 4 or W_u.dim() != 3:
        raise ValueError("q_raw, k_raw, v must be [B, H, T, d] and W_u [r, d, d]")
    B, H, T, d = q_raw.shape
    r = W_u.shape[0]
    dt = q_raw.dtype
    if dt not in _DT or any(x.dtype != dt for x in (k_raw, v, W_u)):
        raise ValueError("q_raw, k_raw, v, W_u must share one dtype: float32 or bfloat16")
    if k_raw.shape != q_raw.shape or v.shape != q_raw.shape or tuple(W_u.shape) != (r, d, d):
        raise ValueError("shape mismatch among q_raw, k_raw, v, W_u")
    if not all(t.is_contiguous() for t in (q_raw, k_raw, v, W_u)):
        raise ValueError("inputs must be contiguous")
    dev = q_raw.device
    for t, shp in ((A0, (B, H, d, d)), (S0, (B, H, d, d)), (n0, (B, H, d))):
        if t is not None:
            _check_out(t, shp, torch.float32, dev, "A0/S0/n0")
    if out is None:
        out = (torch.empty((B, H, T, d), device=dev, dtype=dt), torch.empty((B, H, d, d), device=dev),
               torch.empty((B, H, d, d), device=dev), torch.empty((B, H, d), device=dev),
               torch.empty((B, H, 4), device=dev, dtype=torch.int32))
    o, A_T, S_T, n_T, stats = out
    _check_out(o, (B, H, T, d), dt, dev, "o")
    _check_out(A_T, (B, H, d, d), torch.float32, dev, "A_T")
    _check_out(S_T, (B, H, d, d), torch.float32, dev, "S_T")
    _check_out(n_T, (B, H, d), torch.float32, dev, "n_T")
    if stats is not None:
        _check_out(stats, (B, H, 4), torch.int32, dev, "stats")
    _need_cuda(q_raw, k_raw, v, W_u, A0, S0, n0, o, A_T, S_T, n_T, stats, workspace)
    p = make_params(B, H, T, d, r, dt, eps=eps, nudge_period=nudge_period, s_cap=s_cap, den_eps=den_eps, t0=t0,
                    schedule=schedule, chunk_len=chunk_len, segment_blocks=segment_blocks, update=update)
    lib = _lib.load()
    nbytes = ctypes.c_size_t(0)
    _lib.check(lib.vla_scan_fused_workspace_size(ctypes.byref(p), ctypes.byref(nbytes)))
    ws = workspace
    if nbytes.value and (ws is None or ws.numel() < nbytes.value):
        ws = torch.empty(nbytes.value, device=dev, dtype=torch.uint8)
    with torch.cuda.device(dev):
        _lib.check(lib.vla_scan_forward_fused(
            ctypes.byref(p), _ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(W_u), _ptr(A0), _ptr(S0), _ptr(n0), _ptr(o),
            _ptr(A_T), _ptr(S_T), _ptr(n_T), _ptr(stats), _ptr(ws) if nbytes.value else None, nbytes.value,
            _stream_ptr(dev)))
    return o, A_T, S_T, n_T, stats


def fused_workspace_size(B, H, T, d, r, dtype, **kw) -> int:
    """Bytes of workspace vla_scan_forward_fused needs (0 when the scan kernel runs the prologue)."""
    p = make_params(B, H, T, d, r, dtype, **kw)
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().vla_scan_fused_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def scan_step(q, k, v, u, A, S, n, *, eps=1e-6, nudge_period=0, s_cap=None, den_eps=1e-6, t0=0,
              validate=False, update="additive", o=None, stats=None):
    """Run vla_scan_step: one token per chain (q, k, v [B, H, 1, d], u
    [B, H, 1, r, d]) with the state A, S [B, H, d, d] and n [B, H, d] (float32)
    updated in place.  ``t0`` is the token's global index (nudge phase).
    Returns (o, stats)."""
    _need_cuda(q, k, v, u, A, S, n)
    B, H, T, d = q.shape
    if T != 1:
        raise ValueError("scan_step takes one token per chain (T = 1)")
    r = u.shape[3]
    dt = q.dtype
    if dt not in _DT or any(x.dtype != dt for x in (k, v, u)):
        raise ValueError("q, k, v, u must share one dtype: float32 or bfloat16")
    if k.shape != q.shape or v.shape != q.shape or tuple(u.shape) != (B, H, 1, r, d) or not u.is_contiguous():
        raise ValueError("shape mismatch among q, k, v, u (u contiguous)")
    dev = q.device
    _check_out(A, (B, H, d, d), torch.float32, dev, "A")
    _check_out(S, (B, H, d, d), torch.float32, dev, "S")
    _check_out(n, (B, H, d), torch.float32, dev, "n")
    if o is None:
        o = torch.empty((B, H, 1, d), device=dev, dtype=dt)
    _check_out(o, (B, H, 1, d), dt, dev, "o")
    if stats is None:
        stats = torch.empty((B, H, 4), device=dev, dtype=torch.int32)
    _check_out(stats, (B, H, 4), torch.int32, dev, "stats")
    p = make_params(B, H, 1, d, r, dt, eps=eps, nudge_period=nudge_period, s_cap=s_cap, den_eps=den_eps, t0=t0,
                    validate=validate, update=update, strides=_seq_strides(q, k, v))
    lib = _lib.load()
    ws_bytes = ctypes.c_size_t(0)
    _lib.check(lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(ws_bytes)))
    ws = torch.empty(ws_bytes.value, device=dev, dtype=torch.uint8) if ws_bytes.value else None
    with torch.cuda.device(dev):
        _lib.check(lib.vla_scan_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(A), _ptr(S),
                                     _ptr(n), _ptr(o), _ptr(stats), _ptr(ws), ws_bytes.value, _stream_ptr(dev)))
    return o, stats


def scan_backward(q, k, v, u, A0=None, S0=None, n0=None, *, g_o, g_A=None, g_S=None, g_n=None, eps=1e-6,
                  nudge_period=0, s_cap=None, den_eps=1e-6, t0=0):
    """Run vla_scan_backward: gradients of sum <g_o, o> + <g_A, A_T> + <g_S, S_T>
    + <g_n, n_T> for the additive scan with the same arguments as scan_forward.

    g_o is [B, H, T, d] float32; g_A, g_S, g_n are float32 or None (zero).
    Returns a dict of float32 gradients q, k, v, u, A0, S0, n0."""
    if q.dim() != 4 or u.dim() != 5:
        raise ValueError("q, k, v must be [B, H, T, d] and u [B, H, T, r, d]")
    B, H, T, d = q.shape
    r = u.shape[3]
    dt = q.dtype
    if dt not in _DT or any(x.dtype != dt for x in (k, v, u)):
        raise ValueError("q, k, v, u must share one dtype: float32 or bfloat16")
    if k.shape != q.shape or v.shape != q.shape or tuple(u.shape) != (B, H, T, r, d):
        raise ValueError("shape mismatch among q, k, v, u")
    if not all(t.is_contiguous() for t in (q, k, v, u)):
        raise ValueError("scan_backward takes contiguous inputs")
    dev = q.device
    for t, shp, name in ((A0, (B, H, d, d), "A0"), (S0, (B, H, d, d), "S0"), (n0, (B, H, d), "n0"),
                         (g_o, (B, H, T, d), "g_o"), (g_A, (B, H, d, d), "g_A"), (g_S, (B, H, d, d), "g_S"),
                         (g_n, (B, H, d), "g_n")):
        if t is not None:
            _check_out(t, shp, torch.float32, dev, name)
    _need_cuda(q, k, v, u, A0, S0, n0, g_o, g_A, g_S, g_n)
    p = make_params(B, H, T, d, r, dt, eps=eps, nudge_period=nudge_period, s_cap=s_cap, den_eps=den_eps, t0=t0)
    lib = _lib.load()
    nbytes = ctypes.c_size_t(0)
    _lib.check(lib.vla_scan_backward_workspace_size(ctypes.byref(p), ctypes.byref(nbytes)))
    ws = torch.empty(max(nbytes.value, 1), device=dev, dtype=torch.uint8)
    f32 = dict(device=dev, dtype=torch.float32)
    g = {"q": torch.empty((B, H, T, d), **f32), "k": torch.empty((B, H, T, d), **f32),
         "v": torch.empty((B, H, T, d), **f32), "u": torch.empty((B, H, T, r, d), **f32),
         "A0": torch.empty((B, H, d, d), **f32), "S0": torch.empty((B, H, d, d), **f32),
         "n0": torch.empty((B, H, d), **f32)}
    with torch.cuda.device(dev):
        _lib.check(lib.vla_scan_backward(
            ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(A0), _ptr(S0), _ptr(n0), _ptr(g_o),
            _ptr(g_A), _ptr(g_S), _ptr(g_n), _ptr(g["q"]), _ptr(g["k"]), _ptr(g["v"]), _ptr(g["u"]), _ptr(g["A0"]),
            _ptr(g["S0"]), _ptr(g["n0"]), _ptr(ws), nbytes.value, _stream_ptr(dev)))
    return g


def workspace_size(B, H, T, d, r, dtype, **kw) -> int:
    """Bytes of workspace vla_scan_forward needs (keyword arguments as scan_forward)."""
    p = make_params(B, H, T, d, r, dtype, **kw)
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def project_u(W_u, k_raw, out_dtype=None, out=None):
    """Run vla_project_u: u[..., i, :] = normalize(W_u[i] @ k_raw[...]).

    W_u: [r, d, d]; k_raw: [..., d] (same dtype, float32 or bfloat16).
    Returns u: [..., r, d] in ``out_dtype`` (default: the input dtype).
    """
    _need_cuda(W_u, k_raw)
    if W_u.dim() != 3 or W_u.shape[1] != W_u.shape[2] or k_raw.shape[-1] != W_u.shape[2]:
        raise ValueError("W_u must be [r, d, d] and k_raw [..., d]")
    if W_u.dtype not in _DT or k_raw.dtype != W_u.dtype:
        raise ValueError("W_u and k_raw must share one dtype: float32 or bfloat16")
    if not (W_u.is_contiguous() and k_raw.is_contiguous()):
        raise ValueError("inputs must be contiguous")
    r, d = W_u.shape[0], W_u.shape[1]
    rows = k_raw.numel() // d
    odt = out_dtype or W_u.dtype
    if out is None:
        out = torch.empty(tuple(k_raw.shape[:-1]) + (r, d), device=k_raw.device, dtype=odt)
    lib = _lib.load()
    with torch.cuda.device(k_raw.device):
        _lib.check(lib.vla_project_u(rows, d, r, _DT[W_u.dtype], _DT[odt], _ptr(W_u), _ptr(k_raw), _ptr(out),
                                     _stream_ptr(k_raw.device)))
    return out


def timing_enable(on: bool = True) -> None:
    """Start (or stop) recording HIP events around the state-chain kernel of
    every chunked scan (the library's measurement hook)."""
    _lib.check(_lib.load().vla_timing_enable(1 if on else 0))


def timing_collect() -> list:
    """Durations in ms of the state-chain kernel for the recorded scans, oldest first."""
    lib = _lib.load()
    cap = 256
    buf = (ctypes.c_float * cap)()
    n = ctypes.c_int32(0)
    _lib.check(lib.vla_timing_collect(buf, cap, ctypes.byref(n)))
    return [float(buf[i]) for i in range(n.value)]

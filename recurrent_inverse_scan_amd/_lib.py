"""ctypes view of libvla.so (the C ABI declared in include/vla.h).

Loading never touches the GPU; compute entry points need a HIP device.  The
library is built in-tree by ``recurrent_inverse_scan_amd.build``; if it is
missing, loading fails loudly (there is no fallback implementation).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# VLA_LIB names another build of the same library (the host-sanitised one
# that the CPU test suite makes); by default the in-tree libvla.so.
LIB_PATH = os.environ.get("VLA_LIB") or os.path.join(_PKG, "libvla.so")

VLA_OK, VLA_EINVAL, VLA_EUNSUPPORTED, VLA_EWORKSPACE, VLA_ENONFINITE, VLA_EHIP = range(6)
VLA_F32, VLA_BF16 = 0, 1
VLA_SCHEDULE_AUTO, VLA_SCHEDULE_SEQUENTIAL, VLA_SCHEDULE_CHUNKED = 0, 1, 2
VLA_UPDATE_ADDITIVE, VLA_UPDATE_RESIDUAL = 0, 1
ABI_VERSION = 3
NOALLOC_SCRATCH_BYTES = 256 << 20   # VLA_NOALLOC_SCRATCH_BYTES

# Every symbol include/vla.h declares.
EXPORTED = (
    "vla_scan_params_init", "vla_scan_workspace_size", "vla_scan_forward", "vla_scan_forward_noalloc",
    "vla_scan_step", "vla_scan_backward", "vla_scan_backward_workspace_size", "vla_scan_forward_fused",
    "vla_scan_fused_workspace_size", "vla_project_u",
    "vla_status_string", "vla_last_error", "vla_abi_version", "vla_timing_enable", "vla_timing_collect",
)


class ScanParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
        ("d", ctypes.c_int32), ("r", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("nudge_period", ctypes.c_int32),
        ("s_cap", ctypes.c_float),
        ("den_eps", ctypes.c_float),
        ("t0", ctypes.c_int64),
        ("stride_b", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
        ("stride_t", ctypes.c_int64),
        ("schedule", ctypes.c_int32),
        ("validate", ctypes.c_int32),
        ("chunk_len", ctypes.c_int32),
        ("segment_blocks", ctypes.c_int32),
        ("update", ctypes.c_int32),
        ("para_segments", ctypes.c_int32),
    ]


class VLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libvla.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m recurrent_inverse_scan_amd.build` "
                          "(the VLA scan has no non-HIP implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER(ScanParams)
    lib.vla_scan_params_init.argtypes = [P]
    lib.vla_scan_params_init.restype = None
    lib.vla_scan_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
    lib.vla_scan_workspace_size.restype = i32
    lib.vla_scan_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.vla_scan_forward.restype = i32
    lib.vla_scan_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.vla_scan_forward_noalloc.restype = i32
    lib.vla_scan_backward_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
    lib.vla_scan_backward_workspace_size.restype = i32
    lib.vla_scan_backward.argtypes = [P] + [vp] * 19 + [sz, vp]
    lib.vla_scan_backward.restype = i32
    lib.vla_scan_fused_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
    lib.vla_scan_fused_workspace_size.restype = i32
    lib.vla_scan_forward_fused.argtypes = [P] + [vp] * 13 + [sz, vp]
    lib.vla_scan_forward_fused.restype = i32
    lib.vla_scan_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.vla_scan_step.restype = i32
    lib.vla_project_u.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.vla_project_u.restype = i32
    lib.vla_status_string.argtypes = [i32]
    lib.vla_status_string.restype = ctypes.c_char_p
    lib.vla_last_error.argtypes = []
    lib.vla_last_error.restype = ctypes.c_char_p
    lib.vla_abi_version.argtypes = []
    lib.vla_abi_version.restype = ctypes.c_int
    lib.vla_timing_enable.argtypes = [i32]
    lib.vla_timing_enable.restype = i32
    lib.vla_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32)]
    lib.vla_timing_collect.restype = i32
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != VLA_OK:
        lib = load()
        name = lib.vla_status_string(status).decode()
        detail = lib.vla_last_error().decode()
        raise VLAError(status, f"{name}: {detail}")

"""The C ABI library loads without a GPU, exports every declared symbol, and
rejects bad arguments before launching anything (no compute calls here)."""
import ctypes
import os
import re
import subprocess

import pytest

from recurrent_inverse_scan_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vla.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vla_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libvla.so is not built; run __graft_entry__.build() first")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert set(declared) == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.vla_abi_version() == _lib.ABI_VERSION == 2
    names = [lib.vla_status_string(i).decode() for i in range(6)]
    assert names == ["VLA_OK", "VLA_EINVAL", "VLA_EUNSUPPORTED", "VLA_EWORKSPACE", "VLA_ENONFINITE", "VLA_EHIP"]


def test_timing_collect_rejects_bad_arguments(lib):
    import ctypes

    n = ctypes.c_int32(-1)
    buf = (ctypes.c_float * 4)()
    assert lib.vla_timing_collect(None, 4, ctypes.byref(n)) == _lib.VLA_EINVAL
    assert lib.vla_timing_collect(buf, 4, None) == _lib.VLA_EINVAL
    assert lib.vla_timing_collect(buf, -1, ctypes.byref(n)) == _lib.VLA_EINVAL
    # nothing recorded: an empty, successful collection that needs no device
    assert lib.vla_timing_collect(buf, 4, ctypes.byref(n)) == _lib.VLA_OK and n.value == 0


def test_params_struct_layout_matches_header(lib, tmp_path):
    """The ctypes mirror of vla_scan_params_t has the C compiler's size and
    offsets, and vla_scan_params_init writes the header's defaults."""
    fields = [f for f, _ in _lib.ScanParams._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "vla.h"\nint main(void) {\n'
                   '  printf("%zu", sizeof(vla_scan_params_t));\n'
                   + "".join(f'  printf(" %zu", offsetof(vla_scan_params_t, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    c_layout = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    py_layout = [ctypes.sizeof(_lib.ScanParams)] + [getattr(_lib.ScanParams, f).offset for f in fields]
    assert c_layout == py_layout
    p = _lib.ScanParams()
    ctypes.memset(ctypes.byref(p), 0x5A, ctypes.sizeof(p))
    lib.vla_scan_params_init(ctypes.byref(p))
    assert (p.B, p.H, p.T, p.d, p.r, p.in_dtype) == (0, 0, 0, 64, 1, 0)
    assert abs(p.eps - 1e-6) < 1e-12 and abs(p.den_eps - 1e-6) < 1e-12
    assert (p.nudge_period, p.s_cap, p.t0, p.schedule, p.validate, p.chunk_len) == (0, 0.0, 0, 0, 0, 0)
    assert p.segment_blocks == 0 and p.update == _lib.VLA_UPDATE_ADDITIVE


def _params(lib, **kw):
    p = _lib.ScanParams()
    lib.vla_scan_params_init(ctypes.byref(p))
    p.B, p.H, p.T, p.d, p.r = 1, 1, 4, 64, 1
    for k_, v_ in kw.items():
        setattr(p, k_, v_)
    return p


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every case below fails validation first


def _scan(lib, p, **ptrs):
    args = {n: FAKE for n in ("q", "k", "v", "u", "o", "A_T", "S_T", "n_T")}
    args.update(ptrs)
    return lib.vla_scan_forward(ctypes.byref(p), args["q"], args["k"], args["v"], args["u"], None, None, None,
                                args["o"], args["A_T"], args["S_T"], args["n_T"], None, None, 0, None)


@pytest.mark.parametrize("field,value,status", [
    ("d", 48, _lib.VLA_EUNSUPPORTED), ("d", 256, _lib.VLA_EUNSUPPORTED),
    ("r", 0, _lib.VLA_EUNSUPPORTED), ("r", 5, _lib.VLA_EUNSUPPORTED),
    ("in_dtype", 7, _lib.VLA_EUNSUPPORTED), ("T", -1, _lib.VLA_EINVAL), ("B", -2, _lib.VLA_EINVAL),
    ("nudge_period", -1, _lib.VLA_EINVAL), ("eps", float("nan"), _lib.VLA_EINVAL),
    ("eps", -1.0, _lib.VLA_EINVAL), ("s_cap", float("nan"), _lib.VLA_EINVAL), ("t0", -5, _lib.VLA_EINVAL),
    ("schedule", 9, _lib.VLA_EUNSUPPORTED), ("chunk_len", -3, _lib.VLA_EINVAL),
    ("update", 2, _lib.VLA_EUNSUPPORTED), ("update", -1, _lib.VLA_EUNSUPPORTED),
])
def test_scan_rejects_bad_params(lib, field, value, status):
    p = _params(lib, **{field: value})
    assert _scan(lib, p) == status
    assert lib.vla_last_error().decode() != ""


def test_scan_rejects_null_and_misaligned_pointers(lib):
    p = _params(lib)
    assert _scan(lib, p, q=None) == _lib.VLA_EINVAL
    assert _scan(lib, p, A_T=None) == _lib.VLA_EINVAL
    assert _scan(lib, p, k=ctypes.c_void_p(0x100004)) == _lib.VLA_EINVAL
    assert lib.vla_scan_forward(None, None, None, None, None, None, None, None, None, None, None, None, None,
                                None, 0, None) == _lib.VLA_EINVAL


def test_scan_rejects_overlapping_buffers(lib):
    p = _params(lib)   # 1 chain, T = 4, d = 64, f32: every sequence buffer is 1 KiB
    assert _scan(lib, p, o=ctypes.c_void_p(0x100000)) == _lib.VLA_EINVAL          # o == q
    assert _scan(lib, p, o=ctypes.c_void_p(0x200000), A_T=ctypes.c_void_p(0x200200)) == _lib.VLA_EINVAL


def test_empty_batch_is_a_no_op(lib):
    p = _params(lib, B=0)
    assert lib.vla_scan_forward(ctypes.byref(p), None, None, None, None, None, None, None, None, None, None,
                                None, None, None, 0, None) == _lib.VLA_OK


def test_workspace_size(lib):
    n = ctypes.c_size_t(123)
    p = _params(lib)
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value == 0
    p.validate = 1
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value > 0
    assert _scan(lib, p, o=ctypes.c_void_p(0x300000), A_T=ctypes.c_void_p(0x400000),
                 S_T=ctypes.c_void_p(0x500000), n_T=ctypes.c_void_p(0x600000)) == _lib.VLA_EWORKSPACE


@pytest.mark.parametrize("rows,d,r,din,dout,status", [
    (-1, 64, 1, 0, 0, _lib.VLA_EINVAL), (10, 40, 1, 0, 0, _lib.VLA_EUNSUPPORTED),
    (10, 64, 0, 0, 0, _lib.VLA_EUNSUPPORTED), (10, 64, 1, 3, 0, _lib.VLA_EUNSUPPORTED),
    (10, 64, 1, 0, 0, _lib.VLA_EINVAL),   # null pointers
    (0, 64, 1, 0, 0, _lib.VLA_OK),        # nothing to do
])
def test_project_rejects_bad_args(lib, rows, d, r, din, dout, status):
    assert lib.vla_project_u(rows, d, r, din, dout, None, None, None, None) == status


def test_chunked_schedule_planning(lib):
    n = ctypes.c_size_t(0)
    # d = 64 with a chunk length dividing the nudge period: supported, needs workspace
    p = _params(lib, B=2, H=8, T=65536, schedule=_lib.VLA_SCHEDULE_CHUNKED, nudge_period=1024)
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value > 0
    big = n.value
    # automatic choice takes it too for few chains and long sequences
    p.schedule = _lib.VLA_SCHEDULE_AUTO
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value == big
    # many chains: automatic choice stays sequential (no workspace)
    p.B, p.T = 64, 512
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value == 0
    # explicit chunked with an incompatible chunk length or head size is refused
    for kw in (dict(chunk_len=96, nudge_period=1024), dict(d=128), dict(t0=100, nudge_period=0)):
        q = _params(lib, B=1, H=2, T=4096, schedule=_lib.VLA_SCHEDULE_CHUNKED, **kw)
        assert lib.vla_scan_workspace_size(ctypes.byref(q), ctypes.byref(n)) == _lib.VLA_EUNSUPPORTED


def test_residual_update_schedules(lib):
    """The residual update plans like the additive one: AUTO chunks few long
    chains at d = 64 (with its own state-pass buffers), stays sequential for
    many chains, and an explicit CHUNKED request at d = 128 is refused."""
    n = ctypes.c_size_t(7)
    p = _params(lib, B=2, H=8, T=65536, nudge_period=1024, update=_lib.VLA_UPDATE_RESIDUAL)
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value > 0
    auto = n.value
    p.schedule = _lib.VLA_SCHEDULE_CHUNKED
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value == auto
    p.update = _lib.VLA_UPDATE_ADDITIVE
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value != auto
    q = _params(lib, B=64, H=8, T=512, update=_lib.VLA_UPDATE_RESIDUAL)
    assert lib.vla_scan_workspace_size(ctypes.byref(q), ctypes.byref(n)) == _lib.VLA_OK and n.value == 0
    q = _params(lib, B=1, H=2, T=4096, d=128, schedule=_lib.VLA_SCHEDULE_CHUNKED, update=_lib.VLA_UPDATE_RESIDUAL)
    assert lib.vla_scan_workspace_size(ctypes.byref(q), ctypes.byref(n)) == _lib.VLA_EUNSUPPORTED

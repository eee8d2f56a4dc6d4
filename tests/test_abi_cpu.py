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
    assert lib.vla_abi_version() == _lib.ABI_VERSION == 3
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
    assert (p.stride_b, p.stride_h, p.stride_t) == (0, 0, 0)


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


def test_d128_schedule_choice(lib):
    """At d = 128 the time-parallel schedule needs bf16 storage, the additive
    update and no cap (its state pass is a plain prefix sum); AUTO takes it
    for the wide shape (128 chains of 8192 tokens, rank 4, nudge every 512)
    and sizes its workspace from the per-chunk matrices and coefficients."""
    n = ctypes.c_size_t(7)
    wide = dict(B=8, H=16, T=8192, d=128, r=4, in_dtype=_lib.VLA_BF16, nudge_period=512)
    p = _params(lib, **wide)
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK
    C, T, d, L, P = 128, 8192, 128, 512, 512
    nch, ncs, nper = T // L, T // 256, T // P
    floor = C * d * d * (4 * nch + 8 * nch + 8 * nper + 16 * nper + 4 * nch + 4 * (T // 256)) + C * T * d * 4
    assert n.value >= floor and n.value < floor + (64 << 20)
    auto = n.value
    p.schedule = _lib.VLA_SCHEDULE_CHUNKED
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value == auto
    p.chunk_len = 256
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value > auto
    # sequential otherwise: fp32 storage, a cap, the residual update, or a forced choice
    for kw in (dict(in_dtype=_lib.VLA_F32), dict(s_cap=1e3), dict(update=_lib.VLA_UPDATE_RESIDUAL)):
        q = _params(lib, **{**wide, **kw})
        assert lib.vla_scan_workspace_size(ctypes.byref(q), ctypes.byref(n)) == _lib.VLA_OK and n.value == 0
        q.schedule = _lib.VLA_SCHEDULE_CHUNKED
        assert lib.vla_scan_workspace_size(ctypes.byref(q), ctypes.byref(n)) == _lib.VLA_EUNSUPPORTED
    q = _params(lib, **{**wide, "schedule": _lib.VLA_SCHEDULE_SEQUENTIAL})
    assert lib.vla_scan_workspace_size(ctypes.byref(q), ctypes.byref(n)) == _lib.VLA_OK and n.value == 0


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


# --------------------------------------------------------------------------
# Strided q, k, v (element strides over batch, head and token; d contiguous).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("strides,status", [
    ((-64, 64, 64), _lib.VLA_EINVAL),          # negative
    ((4096, 64, 32), _lib.VLA_EINVAL),         # stride_t < d with T > 1
    ((4096, 66, 64), _lib.VLA_EINVAL),         # 66 * 4 bytes is not a multiple of 16
    ((1 << 60, 64, 64), _lib.VLA_EUNSUPPORTED),
])
def test_scan_rejects_bad_strides(lib, strides, status):
    p = _params(lib, stride_b=strides[0], stride_h=strides[1], stride_t=strides[2])
    assert _scan(lib, p) == status
    assert lib.vla_last_error().decode() != ""


def test_strided_inputs_need_gather_workspace(lib):
    """Strided views are gathered into the workspace: the sequential schedule
    then needs 3 * B*H*T*d elements of it, and the extent a strided view spans
    counts in the overlap checks."""
    n = ctypes.c_size_t(0)
    B, H, T, d = 2, 3, 5, 64
    p = _params(lib, B=B, H=H, T=T, d=d)
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value == 0
    # q from a packed [B, T, H, 3d] float32 projection
    p.stride_b, p.stride_h, p.stride_t = T * H * 3 * d, 3 * d, H * 3 * d
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK
    assert n.value >= 3 * B * H * T * d * 4
    p.in_dtype = _lib.VLA_BF16
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK
    assert 3 * B * H * T * d * 2 <= n.value < 3 * B * H * T * d * 4
    # no workspace given: refused before any launch
    p.in_dtype = _lib.VLA_F32
    assert _scan(lib, p, o=ctypes.c_void_p(0x7000000), A_T=ctypes.c_void_p(0x7100000),
                 S_T=ctypes.c_void_p(0x7200000), n_T=ctypes.c_void_p(0x7300000)) == _lib.VLA_EWORKSPACE
    # o inside the span of a strided q (between its rows) overlaps it
    span = ((B - 1) * p.stride_b + (H - 1) * p.stride_h + (T - 1) * p.stride_t + d) * 4
    assert span > B * H * T * d * 4
    q0 = 0x10000000
    ptrs = dict(q=ctypes.c_void_p(q0), k=ctypes.c_void_p(0x20000000), v=ctypes.c_void_p(0x30000000),
                u=ctypes.c_void_p(0x40000000), A_T=ctypes.c_void_p(0x7100000), S_T=ctypes.c_void_p(0x7200000),
                n_T=ctypes.c_void_p(0x7300000))
    assert _scan(lib, p, o=ctypes.c_void_p(q0 + span - 256), **ptrs) == _lib.VLA_EINVAL
    assert "overlaps" in lib.vla_last_error().decode()
    # just past the span: the aliasing checks pass and the missing workspace is what stops it
    assert _scan(lib, p, o=ctypes.c_void_p(q0 + span), **ptrs) == _lib.VLA_EWORKSPACE


def _step(lib, p, A=FAKE, S=FAKE, n=FAKE, **ptrs):
    args = {x: FAKE for x in ("q", "k", "v", "u", "o")}
    args.update(ptrs)
    return lib.vla_scan_step(ctypes.byref(p), args["q"], args["k"], args["v"], args["u"], A, S, n, args["o"],
                             None, None, 0, None)


def test_scan_step_validates_before_launching(lib):
    """vla_scan_step takes exactly one token and an in-place state."""
    p = _params(lib, T=4)
    assert _step(lib, p) == _lib.VLA_EINVAL and "T = 1" in lib.vla_last_error().decode()
    p = _params(lib, T=1)
    assert _step(lib, p, A=None) == _lib.VLA_EINVAL
    assert _step(lib, p, n=None) == _lib.VLA_EINVAL
    assert lib.vla_scan_step(None, None, None, None, None, None, None, None, None, None, None, 0,
                             None) == _lib.VLA_EINVAL
    p = _params(lib, T=1, d=48)
    assert _step(lib, p) == _lib.VLA_EUNSUPPORTED
    p = _params(lib, T=1, B=0)
    assert lib.vla_scan_step(ctypes.byref(p), None, None, None, None, None, None, None, None, None, None, 0,
                             None) == _lib.VLA_OK


# --------------------------------------------------------------------------
# The Python binding checks caller-supplied outputs and workspace before it
# reaches the C ABI (the library sizes every write from the parameters, so a
# wrong buffer would otherwise be written out of bounds).  CPU tensors stand
# in for device ones: the shape, dtype and layout checks come first.
# --------------------------------------------------------------------------
def _cpu_args(B=1, H=2, T=3, d=16, r=1, dt=None):
    import torch

    dt = dt or torch.float32
    q = torch.zeros(B, H, T, d, dtype=dt)
    u = torch.zeros(B, H, T, r, d, dtype=dt)
    outs = [torch.zeros(B, H, T, d, dtype=dt), torch.zeros(B, H, d, d), torch.zeros(B, H, d, d),
            torch.zeros(B, H, d), torch.zeros(B, H, 4, dtype=torch.int32)]
    return q, u, outs


@pytest.mark.parametrize("which,bad,msg", [
    (0, "bf16", "o must be"), (0, "shape", "o must be"), (1, "shape", "A_T must be"), (1, "f64", "A_T must be"),
    (2, "noncontig", "S_T must be"), (3, "shape", "n_T must be"), (4, "i64", "stats must be"),
    (4, "shape", "stats must be"),
])
def test_binding_rejects_bad_out_tensors(which, bad, msg):
    import torch

    from recurrent_inverse_scan_amd import scan_forward

    q, u, outs = _cpu_args()
    t = outs[which]
    if bad == "bf16":
        t = t.to(torch.bfloat16)
    elif bad == "shape":
        t = t.reshape(-1)[:-1].clone() if t.numel() > 1 else t
    elif bad == "f64":
        t = t.double()
    elif bad == "i64":
        t = t.long()
    elif bad == "noncontig":
        t = t.transpose(-1, -2)
    outs[which] = t
    with pytest.raises(ValueError, match=msg):
        scan_forward(q, q, q, u, out=tuple(outs))


def test_binding_rejects_bad_workspace_and_mixed_strides():
    import torch

    from recurrent_inverse_scan_amd import scan_forward

    q, u, outs = _cpu_args()
    with pytest.raises(ValueError, match="workspace"):
        scan_forward(q, q, q, u, out=tuple(outs), workspace=torch.zeros(64, dtype=torch.float32))
    packed = torch.zeros(1, 3, 2, 48)                  # [B, T, H, 3d]
    qs = packed[..., :16].permute(0, 2, 1, 3)          # strided [B, H, T, d] views
    with pytest.raises(ValueError, match="share their strides"):
        scan_forward(qs, q, q, u)                       # q strided, k and v contiguous
    # well-formed CPU tensors reach the device check last
    with pytest.raises(ValueError, match="HIP device"):
        scan_forward(qs, packed[..., 16:32].permute(0, 2, 1, 3), packed[..., 32:].permute(0, 2, 1, 3), u)


# --------------------------------------------------------------------------
# vla_scan_backward: argument checks before any launch.
# --------------------------------------------------------------------------
def _bwd(lib, p, ws=None, nbytes=0, **ptrs):
    names = ("q", "k", "v", "u", "A0", "S0", "n0", "g_o", "g_AT", "g_ST", "g_nT",
             "g_q", "g_k", "g_v", "g_u", "g_A0", "g_S0", "g_n0")
    base = 0x10000000
    args = {}
    for i, n in enumerate(names):   # distinct, non-overlapping fake addresses
        args[n] = ctypes.c_void_p(base + i * 0x1000000)
    for n in ("A0", "S0", "n0", "g_AT", "g_ST", "g_nT"):
        args[n] = None
    args.update(ptrs)
    return lib.vla_scan_backward(ctypes.byref(p), *[args[n] for n in names], ws, nbytes, None)


def test_backward_workspace_and_supported_set(lib):
    n = ctypes.c_size_t(0)
    p = _params(lib, B=2, H=3, T=100, d=64, r=2)
    assert lib.vla_scan_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value > 0
    # z (r d) + delta, fire (2r) + alpha_hat (d) + |alpha|, c (2) floats per token at least
    assert n.value >= 2 * 3 * 100 * (2 * 64 + 4 + 64 + 2) * 4
    for kw, status in ((dict(d=128), _lib.VLA_EUNSUPPORTED), (dict(update=_lib.VLA_UPDATE_RESIDUAL), _lib.VLA_EUNSUPPORTED),
                       (dict(stride_b=0, stride_h=64, stride_t=64), _lib.VLA_EUNSUPPORTED), (dict(r=7), _lib.VLA_EUNSUPPORTED)):
        q = _params(lib, **{**dict(B=2, H=3, T=100, d=64, r=1), **kw})
        assert lib.vla_scan_backward_workspace_size(ctypes.byref(q), ctypes.byref(n)) == status
        assert _bwd(lib, q) == status


def test_backward_rejects_bad_pointers_and_workspace(lib):
    p = _params(lib, B=1, H=2, T=10, d=32, r=1)
    assert _bwd(lib, p, g_o=None) == _lib.VLA_EINVAL
    assert _bwd(lib, p, g_A0=None) == _lib.VLA_EINVAL
    assert _bwd(lib, p, g_k=ctypes.c_void_p(0x10000000 + 1 * 0x1000000 + 4)) == _lib.VLA_EINVAL   # g_k inside k
    assert _bwd(lib, p, g_v=ctypes.c_void_p(0x10000000 + 11 * 0x1000000)) == _lib.VLA_EINVAL      # g_v == g_q
    assert _bwd(lib, p) == _lib.VLA_EWORKSPACE
    assert "workspace" in lib.vla_last_error().decode()


def test_chunked_schedule_grid_limit(lib):
    """The chunked kernels launch a workgroup per 64-token block of every chain:
    up to 2^22 blocks are planned, beyond that only the sequential schedule runs."""
    n = ctypes.c_size_t(0)
    p = _params(lib, B=1, H=1, T=64 * (1 << 22), schedule=_lib.VLA_SCHEDULE_CHUNKED, nudge_period=0)
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value > 0
    p.T += 64
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_EUNSUPPORTED
    p.schedule = _lib.VLA_SCHEDULE_AUTO
    assert lib.vla_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.VLA_OK and n.value == 0

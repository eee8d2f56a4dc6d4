"""The no-allocation entry point (vla_scan_forward_noalloc) against the
allocating one (vla_scan_forward), through the C ABI.

Two calls in a row share the device's static scratch: a larger chunked
scan, then a smaller one (so the second call runs on what the first left
in the scratch), then a strided sequential call that also needs scratch.
Each must equal vla_scan_forward with a fresh workspace bit for bit and
match the oracle to the parity bar.  The refusal of a call that needs more
scratch than the library holds is checked without a GPU.
"""
import ctypes
import sys

import pytest
import torch

from recurrent_inverse_scan_amd import CONFIGS, scan_forward, workspace_size
from recurrent_inverse_scan_amd import _lib
from recurrent_inverse_scan_amd.api import make_params, scan_forward_noalloc
from tests.parity import case, check, run_oracle

DEV = torch.device("cuda:0")


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _outs(cfg, dtype):
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    return (torch.full((B, H, T, d), float("nan"), device=DEV, dtype=dtype),
            torch.full((B, H, d, d), float("nan"), device=DEV), torch.full((B, H, d, d), float("nan"), device=DEV),
            torch.full((B, H, d), float("nan"), device=DEV), torch.full((B, H, 4), -7, device=DEV, dtype=torch.int32))


CALLS = [
    # (name, overrides, scan keywords): the second is smaller than the first
    ("chunked-larger", dict(B=1, H=3, T=1500, in_dtype="bf16", nudge_period=128, s_cap=30.0),
     dict(schedule="chunked", chunk_len=64, segment_blocks=4)),
    ("chunked-smaller", dict(B=1, H=2, T=700, in_dtype="f32", nudge_period=64, s_cap=25.0),
     dict(schedule="chunked", chunk_len=64)),
]


@pytest.mark.gpu
def test_noalloc_matches_allocating_entry_point_twice_in_a_row():
    for name, over, kw in CALLS:
        cfg = CONFIGS["base"].with_(name=f"noalloc-{name}", **over)
        _say(f"case {name} B={cfg.B} H={cfg.H} T={cfg.T} {cfg.in_dtype} {kw}")
        dt = torch.bfloat16 if cfg.in_dtype == "bf16" else torch.float32
        need = workspace_size(cfg.B, cfg.H, cfg.T, cfg.d, cfg.r, dt, nudge_period=cfg.nudge_period,
                              s_cap=cfg.s_cap, **kw)
        assert 0 < need <= _lib.NOALLOC_SCRATCH_BYTES
        x = case(cfg, seed=70)
        q, k, v, u = (x[n].to(DEV) for n in ("q", "k", "v", "u"))
        want = scan_forward(q, k, v, u, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, **kw)
        got = scan_forward_noalloc(q, k, v, u, out=_outs(cfg, dt), nudge_period=cfg.nudge_period,
                                   s_cap=cfg.s_cap, **kw)
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a, b), name
        check(f"no-alloc/{name}", cfg, got, run_oracle(x, cfg), say=_say)
    # strided q, k, v on the sequential schedule also take their gather from the scratch
    cfg = CONFIGS["base"].with_(name="noalloc-strided", B=2, H=2, T=90, nudge_period=16, s_cap=20.0)
    x = case(cfg, seed=71)
    d = cfg.d
    packed = torch.cat([x["q"], x["k"], x["v"]], dim=-1).permute(0, 2, 1, 3).contiguous().to(DEV)
    qs, ks, vs = (packed[..., i * d:(i + 1) * d].permute(0, 2, 1, 3) for i in range(3))
    got = scan_forward_noalloc(qs, ks, vs, x["u"].to(DEV), out=_outs(cfg, torch.float32),
                               nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, schedule="sequential")
    want = scan_forward(qs, ks, vs, x["u"].to(DEV), nudge_period=cfg.nudge_period, s_cap=cfg.s_cap,
                        schedule="sequential")
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        assert torch.equal(a, b)
    check("no-alloc/strided", cfg, got, run_oracle(x, cfg), say=_say)


def test_noalloc_refuses_calls_beyond_its_scratch():
    """16 chains of 65536 tokens on the chunked schedule need about 1.2 GB of
    workspace: refused with VLA_EWORKSPACE before any launch (no GPU needed)."""
    lib = _lib.load()
    p = make_params(2, 8, 65536, 64, 1, torch.bfloat16, nudge_period=1024, s_cap=1e3, schedule="chunked")
    fake = ctypes.c_void_p(0x100000)
    st = lib.vla_scan_forward_noalloc(ctypes.byref(p), fake, fake, fake, fake, None, None, None, fake, fake, fake,
                                      fake, None, None)
    assert st == _lib.VLA_EWORKSPACE
    assert "vla_scan_forward_noalloc holds" in lib.vla_last_error().decode()

"""GPU parity of the fused entry point (vla_scan_forward_fused): the scan from
raw q, k and W_u, with the feature map and the projection computed by the
library (in the scan kernel itself on the two-wave sequential path).

The reference is the oracle on the composition the entry point is defined
as: q, k = ELU(raw) + 1 in float32 and u = normalize(W_u[i] k_raw) in float64,
each rounded to the storage dtype, then the scan.  Bars as for the scan:
2e-3 (float32 storage) and 1e-2 (bfloat16) normwise.
"""
import sys

import numpy as np
import pytest
import torch

from oracle.vla_oracle import oracle_project_u, oracle_scan
from recurrent_inverse_scan_amd import CONFIGS, fused_workspace_size, make_inputs, scan_forward, scan_forward_fused
from recurrent_inverse_scan_amd.inputs import storage_dtype
from tests.parity import check, rel_err

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(msg):
    print(f"[gpu-fused] {msg}", flush=True)
    sys.stdout.flush()


def _composed(x, cfg, chains=None):
    """q, k, u as the unfused path would store them (CPU side of the test)."""
    dt = storage_dtype(cfg.in_dtype)
    C, T, d, r = cfg.B * cfg.H, cfg.T, cfg.d, cfg.r
    sel = list(range(C)) if chains is None else list(chains)
    feat = lambda raw: (torch.nn.functional.elu(raw.float()) + 1.0).to(dt)
    q = feat(x["q_raw"].reshape(C, T, d)[sel])
    k = feat(x["k_raw"].reshape(C, T, d)[sel])
    u = torch.from_numpy(oracle_project_u(x["W_u"], x["k_raw"].reshape(C, T, d)[sel].reshape(-1, d)))
    u = u.to(dt).reshape(len(sel), T, r, d)
    return q, k, x["v"].reshape(C, T, d)[sel], u


def _fused(x, cfg, **kw):
    args = dict(nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
    args.update(kw)
    out = scan_forward_fused(x["q_raw"].to(DEV), x["k_raw"].to(DEV), x["v"].to(DEV), x["W_u"].to(DEV), **args)
    torch.cuda.synchronize()
    return out


def _ref(x, cfg, chains=None, **kw):
    q, k, v, u = _composed(x, cfg, chains)
    args = dict(nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, trace_norms=True)
    args.update(kw)
    return oracle_scan(q, k, v, u, **args)


# The two-wave kernel builds the features and u in LDS: d <= 64, T > 16.
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,r", [(16, 1), (16, 4), (32, 2), (64, 1), (64, 3), (64, 4)])
def test_fused_in_kernel_matches_oracle(d, r, dtype):
    cfg = CONFIGS["base"].with_(name=f"fused-d{d}-r{r}-{dtype}", B=1, H=3, T=77, d=d, r=r, in_dtype=dtype,
                                nudge_period=6, s_cap=8.0)
    x = make_inputs(cfg, seed=100 + d + r)
    assert fused_workspace_size(cfg.B, cfg.H, cfg.T, d, r, storage_dtype(dtype), nudge_period=6, s_cap=8.0) == 0
    out = _fused(x, cfg)
    check(cfg.name, cfg, out, _ref(x, cfg), say=_say)


@pytest.mark.parametrize("update", ["additive", "residual"])
def test_fused_in_kernel_from_a_state_with_offset(update):
    cfg = CONFIGS["base"].with_(name=f"fused-state-{update}", B=2, H=2, T=45, nudge_period=4, s_cap=20.0)
    x = make_inputs(cfg, seed=7)
    g = torch.Generator().manual_seed(3)
    d = cfg.d
    X = torch.randn(cfg.B, cfg.H, d, d, generator=g) / d
    A0 = (0.6 * torch.eye(d) + X @ X.transpose(-1, -2)).contiguous()
    S0 = torch.randn(cfg.B, cfg.H, d, d, generator=g)
    n0 = torch.rand(cfg.B, cfg.H, d, generator=g)
    out = _fused(x, cfg, A0=A0.to(DEV), S0=S0.to(DEV), n0=n0.to(DEV), t0=5, update=update)
    C = cfg.B * cfg.H
    ref = _ref(x, cfg, A0=A0.reshape(C, d, d), S0=S0.reshape(C, d, d), n0=n0.reshape(C, d), t0=5, update=update)
    check(cfg.name, cfg, out, ref, say=_say)


# Shapes the prologue pass serves: d = 128, the chunked schedule, short calls.
@pytest.mark.parametrize("name,over,kw", [
    ("d128-r4-bf16", dict(B=1, H=2, T=40, d=128, r=4, in_dtype="bf16", nudge_period=8, s_cap=None), {}),
    ("chunked-bf16", dict(B=1, H=2, T=700, in_dtype="bf16", nudge_period=64, s_cap=30.0),
     dict(schedule="chunked", chunk_len=64)),
    ("chunked-f32", dict(B=1, H=2, T=500, in_dtype="f32", nudge_period=128, s_cap=25.0),
     dict(schedule="chunked", chunk_len=64)),
    ("short-T5", dict(B=2, H=3, T=5, in_dtype="f32", nudge_period=2, s_cap=6.0), {}),
    ("decode-T1", dict(B=4, H=4, T=1, in_dtype="bf16", nudge_period=0, s_cap=None), {}),
])
def test_fused_prologue_pass_matches_oracle(name, over, kw):
    cfg = CONFIGS["base"].with_(name=f"fused-{name}", **over)
    x = make_inputs(cfg, seed=11)
    assert fused_workspace_size(cfg.B, cfg.H, cfg.T, cfg.d, cfg.r, storage_dtype(cfg.in_dtype),
                                nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, **kw) > 0
    out = _fused(x, cfg, **kw)
    check(cfg.name, cfg, out, _ref(x, cfg), say=_say)


def test_fused_equals_the_composition_on_the_gpu():
    """The fused kernel and the unfused scan on GPU-projected u agree to
    float32 rounding (bf16 o: one rounding step)."""
    from recurrent_inverse_scan_amd import project_u

    cfg = CONFIGS["recall"].with_(name="fused-vs-unfused", B=4, H=8)
    x = make_inputs(cfg, seed=0)
    a = _fused(x, cfg)
    q, k, v, _ = _composed(x, cfg)
    u = project_u(x["W_u"].to(DEV), x["k_raw"].to(DEV))
    C = cfg.B * cfg.H
    shp = (cfg.B, cfg.H, cfg.T, cfg.d)
    b = scan_forward(q.reshape(shp).to(DEV), k.reshape(shp).to(DEV), v.reshape(shp).to(DEV), u,
                     nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
    torch.cuda.synchronize()
    for name, p_, q_ in zip("oASn", a[:4], b[:4]):
        axes = (-2, -1) if name in "AS" else (-1,)
        err = rel_err(p_.reshape((C,) + tuple(p_.shape[2:])), q_.reshape((C,) + tuple(q_.shape[2:])).cpu().numpy(),
                      axes=axes)
        _say(f"fused vs unfused {name}: {err}")
        assert err <= 1e-4, (name, err)


@pytest.mark.parametrize("name,chains", [("recall", [0, 511]), ("long", [0, 15]), ("wide", [0, 127])])
def test_fused_full_size_sampled_chains(name, chains):
    """Full-size workloads through the fused entry point: recall in the scan
    kernel, long (chunked) and wide (d = 128) through the prologue pass."""
    cfg = CONFIGS[name]
    _say(f"case full/{name} chains={chains}")
    x = make_inputs(cfg, seed=0)
    out = _fused(x, cfg)
    check(f"fused-full-{name}", cfg, out, _ref(x, cfg, chains), chains=chains, say=_say)

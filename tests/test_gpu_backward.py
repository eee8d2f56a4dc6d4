"""GPU parity of the backward pass (vla_scan_backward) against the fp64
gradient oracle (oracle_scan_grad), through the C ABI.

The bar is the normwise relative error per chain and per gradient tensor,
max |x - ref| / max |ref| over the chain's entries: 2e-3 (the gradients are
float32 for both storage dtypes, and bf16 inputs enter exactly).
"""
import sys

import numpy as np
import pytest
import torch

from oracle.vla_oracle_grad import oracle_scan_grad
from recurrent_inverse_scan_amd import CONFIGS, make_inputs, project_u, scan_backward
from tests.parity import case, log_margins

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
BAR = 2e-3


def _say(msg):
    print(f"[gpu-backward] {msg}", flush=True)
    sys.stdout.flush()


def _chain_err(x, ref, C):
    x = x.detach().float().cpu().numpy().astype(np.float64).reshape(C, -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(C, -1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((np.abs(x - ref).max(axis=1) / den).max())


def _cots(cfg, seed, final=True):
    g = torch.Generator().manual_seed(seed)
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    go = torch.randn(B, H, T, d, generator=g)
    if not final:
        return go, None, None, None
    return go, torch.randn(B, H, d, d, generator=g), torch.randn(B, H, d, d, generator=g), torch.randn(B, H, d, generator=g)


def _run(tag, cfg, x, A0=None, S0=None, n0=None, t0=0, seed=0, final=True, chains=None):
    C = cfg.B * cfg.H
    go, gA, gS, gn = _cots(cfg, seed, final)
    dev = lambda t: None if t is None else t.to(DEV)
    got = scan_backward(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), dev(x["u"]), dev(A0), dev(S0), dev(n0),
                        g_o=go.to(DEV), g_A=dev(gA), g_S=dev(gS), g_n=dev(gn), nudge_period=cfg.nudge_period,
                        s_cap=cfg.s_cap, t0=t0)
    torch.cuda.synchronize()
    sel = list(range(C)) if chains is None else list(chains)

    def pick(t, tail):
        return None if t is None else t.reshape((C,) + tail)[sel]

    d, T, r = cfg.d, cfg.T, cfg.r
    ref = oracle_scan_grad(pick(x["q"], (T, d)), pick(x["k"], (T, d)), pick(x["v"], (T, d)),
                           pick(x["u"], (T, r, d)), pick(A0, (d, d)), pick(S0, (d, d)), pick(n0, (d,)),
                           g_o=pick(go, (T, d)), g_A=pick(gA, (d, d)), g_S=pick(gS, (d, d)), g_n=pick(gn, (d,)),
                           nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, t0=t0)
    tails = {"q": (T, d), "k": (T, d), "v": (T, d), "u": (T, r, d), "A0": (d, d), "S0": (d, d), "n0": (d,)}
    errs = {}
    for name, tail in tails.items():
        g_sel = got[name].reshape((C,) + tail)[sel]
        errs[name] = _chain_err(g_sel, ref[name], len(sel)) if T > 0 or name in ("A0", "S0", "n0") else 0.0
    log_margins(f"backward/{tag}", cfg, errs, {}, {})
    _say(f"{tag}: {errs}")
    assert all(v <= BAR for v in errs.values()), errs
    return got, ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,r", [(16, 1), (32, 3), (64, 1), (64, 2)])
def test_backward_matches_oracle(d, r, dtype):
    """Guard-free SPD start with an offset, nudges, a binding cap, a ragged
    last checkpoint chunk (T = 77 over chunks of 32)."""
    cfg = CONFIGS["base"].with_(name=f"bwd-d{d}-r{r}-{dtype}", B=1, H=3, T=77, d=d, r=r, in_dtype=dtype,
                                nudge_period=5, s_cap=6.0)
    x = case(cfg, seed=80 + d + r)
    g = torch.Generator().manual_seed(d * r)
    C = cfg.B * cfg.H
    X = torch.randn(cfg.B, cfg.H, d, d, generator=g) / d
    A0 = (0.7 * torch.eye(d) + X @ X.transpose(-1, -2)).contiguous()
    S0 = torch.randn(cfg.B, cfg.H, d, d, generator=g)
    n0 = torch.rand(cfg.B, cfg.H, d, generator=g)
    _run(cfg.name, cfg, x, A0, S0, n0, t0=3, seed=d + r)


def test_backward_cap_forced_every_step_and_no_final_cotangents():
    """cap = 1 fires on every token (scales near 0.1): the checkpointed
    recomputation of S keeps the reverse pass exact where undoing the scale
    would amplify rounding."""
    cfg = CONFIGS["base"].with_(name="bwd-cap1", B=1, H=2, T=70, nudge_period=0, s_cap=1.0)
    x = case(cfg, seed=90)
    _run(cfg.name, cfg, x, seed=5, final=False)


def test_backward_guard_fire_gives_no_gradient_to_its_direction():
    cfg = CONFIGS["base"].with_(name="bwd-guard", B=1, H=2, T=20, nudge_period=0, s_cap=None)
    x = case(cfg, seed=91)
    e = torch.zeros(cfg.d)
    e[5] = 1.0
    u = x["u"].clone()
    u[:, :, 0, 0, :] = e
    x["u"] = u
    A0 = (torch.eye(cfg.d) - 2 * torch.outer(e, e)).expand(1, 2, cfg.d, cfg.d).contiguous()
    got, _ = _run(cfg.name, cfg, x, A0=A0, seed=6)
    assert torch.equal(got["u"][:, :, 0, 0].cpu(), torch.zeros(1, 2, cfg.d))


def test_backward_empty_sequence_passes_the_final_cotangents_through():
    cfg = CONFIGS["base"].with_(name="bwd-empty", B=2, H=2, T=0)
    x = case(cfg, seed=92)
    got, ref = _run(cfg.name, cfg, x, seed=7)
    go, gA, gS, gn = _cots(cfg, 7)
    assert torch.equal(got["A0"].cpu(), gA) and torch.equal(got["S0"].cpu(), gS) and torch.equal(got["n0"].cpu(), gn)


@pytest.mark.parametrize("name,chains", [("recall", [0, 511]), ("base", [0, 31])])
def test_backward_full_size_sampled_chains(name, chains):
    """The recall (512 chains x 512 tokens) and base (32 x 2048, nudge and
    cap) workloads at full size on the GPU, u from the GPU projection; the
    oracle checks two chains."""
    cfg = CONFIGS[name]
    _say(f"case full/{name} chains={chains}")
    x = make_inputs(cfg, seed=0)
    u = project_u(x["W_u"].to(DEV), x["k_raw"].to(DEV))
    x = dict(x)
    x["u"] = u.cpu()
    _run(f"full-{name}", cfg, x, seed=8, chains=chains)

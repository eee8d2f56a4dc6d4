"""Helpers shared by the GPU parity tests: inputs, the oracle's side, and the
normwise relative-error measure used as the parity bar."""
import numpy as np
import torch

from oracle.vla_oracle import oracle_project_u, oracle_scan
from recurrent_inverse_scan_amd import make_inputs
from recurrent_inverse_scan_amd.inputs import storage_dtype

# Tolerances on the normwise relative error: fp32 storage 2e-3, bf16 storage 1e-2.
TOL = {"f32": 2e-3, "bf16": 1e-2}


def to64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def rel_err(x, ref, axes=(-1,)):
    """max over leading indices of |x - ref|_inf / |ref|_inf, the max taken over ``axes``.

    Used per output row (axes=(-1,)) and per state matrix (axes=(-2, -1))."""
    x, ref = to64(x), np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    num = np.abs(x - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    floor = 1e-30 + 1e-12 * np.abs(ref).max()
    return float((num / np.maximum(den, floor)).max()) if num.size else 0.0


def oracle_u(W_u, k_raw, cfg):
    """u from the oracle's projection, cast to the storage dtype (round to nearest even)."""
    u64 = oracle_project_u(W_u, k_raw.reshape(-1, cfg.d))
    return torch.from_numpy(u64).to(storage_dtype(cfg.in_dtype)).reshape(cfg.B, cfg.H, cfg.T, cfg.r, cfg.d)


def case(cfg, seed=0):
    """Inputs in the storage dtype plus u from the oracle's projection (shared by both sides)."""
    x = make_inputs(cfg, seed)
    x["u"] = oracle_u(x["W_u"], x["k_raw"], cfg)
    return x


def run_oracle(x, cfg, chains=None, **kw):
    """Oracle on all chains, or on the flat chain indices ``chains``."""
    B, H, T, d, r = cfg.B, cfg.H, cfg.T, cfg.d, cfg.r
    C = B * H

    def pick(t, tail):
        t = t.reshape((C,) + tail)
        return t if chains is None else t[list(chains)]

    args = dict(nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
    args.update(kw)
    return oracle_scan(pick(x["q"], (T, d)), pick(x["k"], (T, d)), pick(x["v"], (T, d)),
                       pick(x["u"], (T, r, d)), **args)


def flat(t, cfg, chains=None, tail=None):
    """GPU result reshaped to [chains, ...] and optionally restricted to ``chains``."""
    t = t.reshape((cfg.B * cfg.H,) + tuple(t.shape[2:]))
    return t if chains is None else t[list(chains)]

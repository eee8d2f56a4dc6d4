"""Helpers shared by the GPU parity tests: inputs, the oracle's side, and the
normwise relative-error measure used as the parity bar."""
import json
import os

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


def elem_err(x, ref):
    """max over entries of |x - ref| / (|ref| + 1e-6 max|ref|): elementwise, for information only."""
    x, ref = to64(x), np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    return float((np.abs(x - ref) / (np.abs(ref) + 1e-6 * np.abs(ref).max() + 1e-300)).max())


def log_margins(tag, cfg, errs, elem, extra=None):
    """Append one case's errors to the JSON-lines file named by VLA_PARITY_LOG (if set)."""
    path = os.environ.get("VLA_PARITY_LOG")
    if not path:
        return
    rec = {"case": tag, "test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], "workload": cfg.name, "B": cfg.B, "H": cfg.H, "T": cfg.T, "d": cfg.d, "r": cfg.r,
           "storage": cfg.in_dtype, "tol": TOL[cfg.in_dtype], "normwise": errs, "elementwise": elem}
    rec.update(extra or {})
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def first_cap_ok(gpu_first, ref, cap, margin=1e-3):
    """Whether each chain's first cap step is one the exact scan allows.

    The oracle's pre-cap norms decide: a step g is admissible when its norm is
    above cap (1 - margin) and no earlier norm exceeds cap (1 + margin); where
    the oracle's norms clear the cap by more than the margin this leaves only
    the oracle's own first step, so the comparison is exact there."""
    pre = ref["pre_cap_norm"]
    ok = []
    for c, g in enumerate(np.asarray(gpu_first).reshape(-1)):
        g = int(g)
        row = pre[c]
        if g < 0:
            ok.append(bool((row <= cap * (1 + margin)).all()))
        else:
            ok.append(bool(g < row.size and row[g] > cap * (1 - margin) and (row[:g] <= cap * (1 + margin)).all()))
    return np.array(ok)


def check(tag, cfg, out, ref, chains=None, tol=None, say=print):
    """Compare a GPU result with the oracle: normwise errors against the bar,
    guard fires and the non-finite flag exactly, cap fires within the
    rounding allowance, and the first cap step (when the oracle traced its
    norms).  Returns (errors, stats as a numpy array)."""
    tol = tol or TOL[cfg.in_dtype]
    o, A, S, n, st = out
    fo, fA, fS, fn = flat(o, cfg, chains), flat(A, cfg, chains), flat(S, cfg, chains), flat(n, cfg, chains)
    errs = {"o": rel_err(fo, ref["o"]), "A": rel_err(fA, ref["A"], axes=(-2, -1)),
            "S": rel_err(fS, ref["S"], axes=(-2, -1)), "n": rel_err(fn, ref["n"])}
    elem = {"o": elem_err(fo, ref["o"]), "A": elem_err(fA, ref["A"]), "S": elem_err(fS, ref["S"]),
            "n": elem_err(fn, ref["n"])}
    st = flat(st, cfg, chains).cpu().numpy()
    extra = {"guard_fires": st[:, 0].tolist(), "cap_fires": st[:, 1].tolist(),
             "oracle_cap_fires": np.asarray(ref["cap_fires"]).tolist(),
             "first_cap_step": st[:, 3].tolist(), "oracle_first_cap_step": np.asarray(ref["first_cap_step"]).tolist()}
    log_margins(tag, cfg, errs, elem, extra)
    say(f"{tag}: {cfg.name} B={cfg.B} H={cfg.H} T={cfg.T} d={cfg.d} r={cfg.r} {cfg.in_dtype}: {errs} elem {elem}")
    assert all(v <= tol for v in errs.values()), errs
    np.testing.assert_array_equal(st[:, 0], ref["guard_fires"])
    assert (st[:, 2] == ref["nonfinite"]).all()
    if cfg.s_cap:
        # cap decisions may differ only where |S|_F is within rounding of the cap
        assert np.abs(st[:, 1] - ref["cap_fires"]).max() <= max(2, 0.01 * ref["cap_fires"].max())
        if "pre_cap_norm" in ref:
            ok = first_cap_ok(st[:, 3], ref, cfg.s_cap)
            assert ok.all(), (st[:, 3], ref["first_cap_step"])
    return errs, st


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

    args = dict(nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, trace_norms=True)
    args.update(kw)
    return oracle_scan(pick(x["q"], (T, d)), pick(x["k"], (T, d)), pick(x["v"], (T, d)),
                       pick(x["u"], (T, r, d)), **args)


def flat(t, cfg, chains=None, tail=None):
    """GPU result reshaped to [chains, ...] and optionally restricted to ``chains``."""
    t = t.reshape((cfg.B * cfg.H,) + tuple(t.shape[2:]))
    return t if chains is None else t[list(chains)]

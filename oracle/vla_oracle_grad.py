"""Plain fp64 CPU oracle for the gradients of the VLA recurrence scan.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only the test suite and the benchmark's ``cpu_baseline``
leg use it.  It shares no code, constants or helpers with the HIP library.

The pages stress that the scan carries "full gradient flow" ("Variational
Linear Attention (VLA)" README, VLA v3 research implementation notes item
2; "Mathematical Primitives" section 5 on keeping the backward pass
stable).  They state the forward recurrence only, so the gradient here is
the exact derivative of that recurrence: the scan is written out once more,
token by token, in float64 torch operations that mirror ``oracle_scan``
step for step (same readings: guard per sub-update with the update skipped
on a fire, nudge after the sub-updates and before alpha, alpha_hat =
alpha / max(|alpha|, 1), S is [value, key], strict cap rescaling to exactly
the cap before the readout, readout from the post-update S_t and n_t), and
torch's reverse-mode differentiation gives the gradient of

    L = sum_t <g_o[t], o_t> + <g_A, A_T> + <g_S, S_T> + <g_n, n_T>

with respect to q, k, v, u, A0, S0 and n0.  The tests pin this against the
float64 NumPy oracle: equal forward values, central finite differences of
``oracle_scan`` itself, and a closed form (linear attention at u = 0).
Only the additive update is covered.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["oracle_scan_grad"]


def _t64(x, torch):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        if x.dtype in (torch.bfloat16, torch.float16):
            x = x.to(torch.float32)
        return x.to(torch.float64).clone()
    return torch.from_numpy(np.asarray(x, dtype=np.float64).copy())


def _scan_torch(torch, q, k, v, u, A, S, n, eps, nudge_period, s_cap, den_eps, t0):
    """The additive scan on [C, ...] float64 tensors; returns o, A_T, S_T, n_T."""
    C, T, d = q.shape
    r = u.shape[2]
    eye = torch.eye(d, dtype=torch.float64)
    cap_on = s_cap is not None and s_cap > 0 and math.isfinite(s_cap)
    outs = []
    for t in range(T):
        for i in range(r):   # r sequential Sherman-Morrison steps with the guard
            ui = u[:, t, i, :]
            z = torch.einsum("cij,cj->ci", A, ui)
            delta = 1.0 + (ui * z).sum(-1)
            fire = delta.abs() < eps
            safe = torch.where(fire, torch.ones_like(delta), delta)
            upd = A - z[:, :, None] * z[:, None, :] / safe[:, None, None]
            A = torch.where(fire[:, None, None], A + eps * eye, upd)
        tau = t0 + t + 1
        if nudge_period > 0 and tau % nudge_period == 0:
            A = A + eps * eye
        alpha = torch.einsum("cij,cj->ci", A, k[:, t, :])
        anorm = torch.sqrt((alpha * alpha).sum(-1))
        alpha_hat = alpha / torch.clamp(anorm, min=1.0)[:, None]
        S = S + v[:, t, :, None] * alpha_hat[:, None, :]
        if cap_on:
            fn = torch.sqrt((S * S).sum((-2, -1)))
            over = fn > s_cap
            scale = torch.where(over, s_cap / torch.where(over, fn, torch.ones_like(fn)), torch.ones_like(fn))
            S = S * scale[:, None, None]
        n = n + k[:, t, :]
        den = (n * q[:, t, :]).sum(-1) + den_eps
        outs.append(torch.einsum("cij,cj->ci", S, q[:, t, :]) / den[:, None])
    o = torch.stack(outs, dim=1) if outs else torch.zeros((C, 0, d), dtype=torch.float64)
    return o, A, S, n


def oracle_scan_grad(q, k, v, u, A0=None, S0=None, n0=None, *, g_o, g_A=None, g_S=None, g_n=None, eps=1e-6,
                     nudge_period=0, s_cap=None, den_eps=1e-6, t0=0):
    """Gradients of L (above) for the additive scan, in float64.

    Shapes as ``oracle_scan``: q, k, v, g_o [*batch, T, d]; u [*batch, T, r, d];
    A0, S0, g_A, g_S [*batch, d, d]; n0, g_n [*batch, d]; None for A0, S0, n0
    means I, 0, 0 and None for a g_* means 0.  Returns a dict of float64
    arrays: the forward results ``o``, ``A``, ``S``, ``n`` and the gradients
    ``q``, ``k``, ``v``, ``u``, ``A0``, ``S0``, ``n0`` (same shapes as the
    corresponding inputs).
    """
    import torch

    q, k, v, u, g_o = (_t64(x, torch) for x in (q, k, v, u, g_o))
    batch = tuple(q.shape[:-2])
    T, d = q.shape[-2], q.shape[-1]
    r = u.shape[-2]
    C = int(np.prod(batch)) if batch else 1
    q, k, v, g_o = (x.reshape(C, T, d) for x in (q, k, v, g_o))
    u = u.reshape(C, T, r, d)
    A = _t64(A0, torch).reshape(C, d, d) if A0 is not None else torch.eye(d, dtype=torch.float64).repeat(C, 1, 1)
    S = _t64(S0, torch).reshape(C, d, d) if S0 is not None else torch.zeros(C, d, d, dtype=torch.float64)
    n = _t64(n0, torch).reshape(C, d) if n0 is not None else torch.zeros(C, d, dtype=torch.float64)
    leaves = [q, k, v, u, A, S, n]
    for x in leaves:
        x.requires_grad_(True)
    o, A_T, S_T, n_T = _scan_torch(torch, q, k, v, u, A, S, n, eps, nudge_period, s_cap, den_eps, t0)
    loss = (o * g_o).sum()
    for out, g, shp in ((A_T, g_A, (C, d, d)), (S_T, g_S, (C, d, d)), (n_T, g_n, (C, d))):
        if g is not None:
            loss = loss + (out * _t64(g, torch).reshape(shp)).sum()
    grads = torch.autograd.grad(loss, leaves, allow_unused=True)
    names = ["q", "k", "v", "u", "A0", "S0", "n0"]
    shapes = [batch + (T, d)] * 3 + [batch + (T, r, d), batch + (d, d), batch + (d, d), batch + (d,)]
    res = {}
    for name, g, x, shp in zip(names, grads, leaves, shapes):
        g = torch.zeros_like(x) if g is None else g
        res[name] = g.detach().numpy().reshape(shp)
    res["o"] = o.detach().numpy().reshape(batch + (T, d))
    res["A"] = A_T.detach().numpy().reshape(batch + (d, d))
    res["S"] = S_T.detach().numpy().reshape(batch + (d, d))
    res["n"] = n_T.detach().numpy().reshape(batch + (d,))
    return res

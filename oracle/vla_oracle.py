"""Plain fp64 CPU oracle for the Variational Linear Attention (VLA) recurrence scan.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only the test suite, the smoke check and the benchmark's
``cpu_baseline`` leg use it.  It shares no code, constants or helpers with the
HIP library, and it imports nothing from it.

Every step is written out the way the pages state it, one token at a time,
vectorised only over independent (batch, head) chains.  All arithmetic is
float64; inputs stored as float32 or bfloat16 are widened exactly.

Sources (pages and sections):

* "Mathematical Primitives" (VLA documentation site)
  - section 2, "Sherman-Morrison Rank-1 Inverse Tracking": the rank-1 inverse
    update, its five-step execution pipeline (z = A u, delta = 1 + u.z, the
    |delta| < eps guard that injects eps*I, A <- A - z z^T / delta) and the
    periodic eps*I spectrum stabilisation;
  - section 3, "The Woodbury Matrix Generalization": rank r processed as r
    sequential rank-1 updates;
  - section 4, "Analytical Optimal Coefficient Recovery": alpha_t = A_t s_t;
  - section 5, "Recurrent State Modulations": the additive state update, the
    batched outer-product idiom that fixes its orientation, and the Frobenius
    renormalisation of S.
* "Variational Linear Attention (VLA)" (project README), "VLA v3 research
  implementation notes": ELU+1 features, u = normalize(W_u k_raw), normalised
  (k, alpha) outer-product updates and the z.q readout denominator.

Readings taken where the pages are silent or ambiguous (each listed with its
reason in the design notes):

* s_t in alpha = A_t s_t is the key feature vector k_t (the scalar score of
  section 1 cannot multiply a matrix); no 1/sqrt(d).
* alpha uses A_t after all r rank-1 updates and after step t's nudge.
* alpha_hat = alpha / max(||alpha||_2, 1).
* S is [value, key]: S_ij += v_i alpha_hat_j; o = S q.
* Guard: per rank-1 sub-update, strict |delta| < eps; on a fire A <- A + eps*I
  and that update is skipped.  Otherwise divide by the signed delta.
* Nudge: A <- A + eps*I when nudge_period > 0 and tau mod nudge_period == 0,
  tau = t0 + t the 1-based global token index; applied after the rank-1
  updates, before alpha.
* Cap: checked every step after the S update and before the readout; strict
  ||S||_F > cap rescales S to exactly cap.  cap None, <= 0 or inf disables it.
* Readout uses the post-update S_t and n_t: o_t = S_t q_t / (n_t . q_t + den_eps).
* normalize(x) = x / max(||x||_2, 1e-12).

The residual (delta-rule) update ("Variational Linear Attention: Stable
Associative Memory for Long-Context Transformers", technical summary 2.3,
recursive update rule) replaces the coefficient and state steps with:

* k_hat = normalize(k_t), alpha_hat = normalize(A_t k_hat), with A_t taken
  after the rank-1 updates and the nudge as above;
* S_t = S_{t-1} + (v_t - S_{t-1} k_hat) alpha_hat^T.

The inverse recurrence, the nudge, the cap and the readout (n accumulates the
raw feature k_t; o_t = S_t q_t / (n_t . q_t + den_eps)) are unchanged.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["oracle_scan", "oracle_project_u", "as_f64"]


def as_f64(x) -> np.ndarray:
    """Widen an array (numpy, or a CPU torch tensor of any float dtype) to float64."""
    if hasattr(x, "detach"):  # a torch tensor: go through float32, which holds bf16 exactly
        import torch

        x = x.detach().to("cpu")
        if x.dtype in (torch.bfloat16, torch.float16):
            x = x.to(torch.float32)
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def _cap_enabled(s_cap) -> bool:
    return s_cap is not None and s_cap > 0 and math.isfinite(s_cap)


def _normalize_rows(x):
    """x / max(||x||_2, 1e-12) along the last axis."""
    nrm = np.sqrt(np.einsum("ci,ci->c", x, x))
    return x / np.maximum(nrm, 1e-12)[:, None]


def oracle_scan(q, k, v, u, A0=None, S0=None, n0=None, *, eps=1e-6, nudge_period=0,
                s_cap=None, den_eps=1e-6, t0=0, update="additive", normalize=True, trace_norms=False):
    """Run the VLA scan sequentially over tokens, independently per chain.

    ``update`` selects the state step: "additive" (S += v alpha_hat^T with the
    clamp alpha_hat = alpha / max(||alpha||, 1)) or "residual" (the delta-rule
    form with unit k_hat and unit alpha_hat).  ``normalize=False`` (residual
    only) drops both unit normalisations, i.e. alpha = A_t k and
    S += (v - S k) alpha^T: the recursive-least-squares form, which has a
    closed form and serves as a check of the residual step.

    Shapes: q, k, v are [*batch, T, d]; u is [*batch, T, r, d] (u[..., t, i, :] is
    the i-th penalty direction of token t, applied in index order).  A0 and S0
    are [*batch, d, d], n0 is [*batch, d]; None means I, 0 and 0.

    Returns a dict with float64 arrays ``o`` [*batch, T, d], ``A`` and ``S``
    [*batch, d, d], ``n`` [*batch, d] and per-chain statistics:
    ``guard_fires``, ``cap_fires``, ``first_cap_step`` (0-based local token
    index, -1 if none), ``max_s_norm`` (largest ||S_t||_F after the cap) and
    ``nonfinite`` (any output or final state not finite).  With
    ``trace_norms`` it also returns ``pre_cap_norm`` [*batch, T], each token's
    ||S_t||_F after the state update and before the cap is applied.
    """
    q, k, v, u = as_f64(q), as_f64(k), as_f64(v), as_f64(u)
    batch = q.shape[:-2]
    T, d = q.shape[-2], q.shape[-1]
    r = u.shape[-2]
    if update not in ("additive", "residual"):
        raise ValueError(f"unknown update {update!r}")
    if not normalize and update != "residual":
        raise ValueError("normalize=False applies to the residual update only")
    if k.shape != q.shape or v.shape != q.shape or u.shape != batch + (T, r, d):
        raise ValueError("shape mismatch among q, k, v, u")
    C = int(np.prod(batch)) if batch else 1
    q = q.reshape(C, T, d)
    k = k.reshape(C, T, d)
    v = v.reshape(C, T, d)
    u = u.reshape(C, T, r, d)

    eye = np.eye(d)
    A = np.broadcast_to(eye, (C, d, d)).copy() if A0 is None else as_f64(A0).reshape(C, d, d).copy()
    S = np.zeros((C, d, d)) if S0 is None else as_f64(S0).reshape(C, d, d).copy()
    n = np.zeros((C, d)) if n0 is None else as_f64(n0).reshape(C, d).copy()

    guard = np.zeros(C, dtype=np.int64)
    capf = np.zeros(C, dtype=np.int64)
    first_cap = np.full(C, -1, dtype=np.int64)
    max_norm = np.zeros(C)
    pre_norm = np.zeros((C, T)) if trace_norms else None
    o = np.zeros((C, T, d))
    cap_on = _cap_enabled(s_cap)

    for t in range(T):
        # Rank-r perturbation as r sequential Sherman-Morrison steps
        # ("Mathematical Primitives", sections 2 and 3).
        for i in range(r):
            ui = u[:, t, i, :]
            z = np.einsum("cij,cj->ci", A, ui)                   # z = A u
            delta = 1.0 + np.einsum("ci,ci->c", ui, z)           # delta = 1 + u.z
            fire = np.abs(delta) < eps                           # singularity guard
            safe = np.where(fire, 1.0, delta)
            upd = A - np.einsum("ci,cj->cij", z, z) / safe[:, None, None]
            A = np.where(fire[:, None, None], A + eps * eye, upd)
            guard += fire
        # Periodic spectrum stabilisation: eps*I added every nudge_period tokens.
        tau = t0 + t + 1
        if nudge_period > 0 and tau % nudge_period == 0:
            A = A + eps * eye
        if update == "additive":
            # Optimal coefficient alpha = A_t k_t, clamped to norm <= 1.
            alpha = np.einsum("cij,cj->ci", A, k[:, t, :])
            anorm = np.sqrt(np.einsum("ci,ci->c", alpha, alpha))
            alpha_hat = alpha / np.maximum(anorm, 1.0)[:, None]
            # Additive fast-weight update S += v alpha_hat^T ([value, key] layout).
            S = S + v[:, t, :, None] * alpha_hat[:, None, :]
        else:
            # Residual update: gating vector from the unit key, and the
            # prediction error of the previous state written along it.
            khat = _normalize_rows(k[:, t, :]) if normalize else k[:, t, :]
            alpha = np.einsum("cij,cj->ci", A, khat)
            alpha_hat = _normalize_rows(alpha) if normalize else alpha
            resid = v[:, t, :] - np.einsum("cij,cj->ci", S, khat)
            S = S + resid[:, :, None] * alpha_hat[:, None, :]
        # Frobenius renormalisation of S.
        fn = np.sqrt(np.einsum("cij,cij->c", S, S))
        if trace_norms:
            pre_norm[:, t] = fn
        if cap_on:
            over = fn > s_cap
            scale = np.where(over, s_cap / np.where(over, fn, 1.0), 1.0)
            S = S * scale[:, None, None]
            first_cap = np.where(over & (first_cap < 0), t, first_cap)
            capf += over
            fn = np.where(over, s_cap, fn)
        max_norm = np.maximum(max_norm, fn)
        # Normaliser and calibrated readout.
        n = n + k[:, t, :]
        den = np.einsum("ci,ci->c", n, q[:, t, :]) + den_eps
        o[:, t, :] = np.einsum("cij,cj->ci", S, q[:, t, :]) / den[:, None]

    nonfinite = ~(np.isfinite(o).all(axis=(1, 2)) & np.isfinite(A).all(axis=(1, 2))
                  & np.isfinite(S).all(axis=(1, 2)) & np.isfinite(n).all(axis=1))
    out = {
        "o": o.reshape(batch + (T, d)),
        "A": A.reshape(batch + (d, d)),
        "S": S.reshape(batch + (d, d)),
        "n": n.reshape(batch + (d,)),
        "guard_fires": guard.reshape(batch),
        "cap_fires": capf.reshape(batch),
        "first_cap_step": first_cap.reshape(batch),
        "max_s_norm": max_norm.reshape(batch),
        "nonfinite": nonfinite.reshape(batch),
    }
    if trace_norms:
        out["pre_cap_norm"] = pre_norm.reshape(batch + (T,))
    return out


def oracle_project_u(W_u, k_raw):
    """Penalty directions u_{.,i} = normalize(W_u[i] k_raw) in float64.

    "Variational Linear Attention (VLA)" README, v3 notes item 2 (learned
    penalty direction).  W_u is [r, d, d] and is applied as a matrix-vector
    product W_u[i] @ k_raw; k_raw is [rows, d].  Returns [rows, r, d].
    normalize(x) = x / max(||x||_2, 1e-12).
    """
    W = as_f64(W_u)
    kr = as_f64(k_raw)
    if W.ndim != 3 or W.shape[1] != W.shape[2] or kr.shape[-1] != W.shape[2]:
        raise ValueError("W_u must be [r, d, d] and k_raw [rows, d]")
    rows = kr.reshape(-1, kr.shape[-1])
    out = np.empty((rows.shape[0], W.shape[0], W.shape[1]))
    for i in range(W.shape[0]):
        x = rows @ W[i].T                      # x[row] = W[i] @ k_raw[row]
        nrm = np.sqrt(np.sum(x * x, axis=1))
        out[:, i, :] = x / np.maximum(nrm, 1e-12)[:, None]
    return out.reshape(kr.shape[:-1] + (W.shape[0], W.shape[1]))

"""Planted mistakes: every plausible slip in the oracle must fail some pin.

Each mutant is a copy of the oracle's source with one deliberate error,
loaded into a fresh module on the CPU.  All pins of ``test_oracle_pins`` are
run against it with the module's oracle names swapped for the mutant's; the
test passes only if at least one pin fails for every mutant.  (Mistakes are
planted in the oracle only, never in GPU code.)
"""
import importlib.util
import os
import types

import pytest

from tests import test_oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "vla_oracle.py")

# (description, original text, replacement): each original occurs exactly once.
MUTANTS = [
    ("rank-1 update with the wrong sign",
     'upd = A - np.einsum("ci,cj->cij", z, z)', 'upd = A + np.einsum("ci,cj->cij", z, z)'),
    ("denominator without the leading 1",
     "delta = 1.0 + np.einsum", "delta = 0.0 + np.einsum"),
    ("z uses the key instead of the penalty direction",
     'z = np.einsum("cij,cj->ci", A, ui)', 'z = np.einsum("cij,cj->ci", A, k[:, t, :])'),
    ("guard on signed delta instead of its magnitude",
     "fire = np.abs(delta) < eps", "fire = delta < eps"),
    ("guard fire does not skip the update",
     "A = np.where(fire[:, None, None], A + eps * eye, upd)",
     "A = np.where(fire[:, None, None], upd + eps * eye, upd)"),
    ("guard injects nothing",
     "A = np.where(fire[:, None, None], A + eps * eye, upd)",
     "A = np.where(fire[:, None, None], A, upd)"),
    ("only the first of r directions applied", "for i in range(r):", "for i in range(min(r, 1)):"),
    ("nudge phase off by one", "tau = t0 + t + 1", "tau = t0 + t"),
    ("nudge ignores the resume offset", "tau = t0 + t + 1", "tau = t + 1"),
    ("nudge adds twice eps", "A = A + eps * eye\n", "A = A + 2 * eps * eye\n"),
    ("alpha from the penalty direction", 'alpha = np.einsum("cij,cj->ci", A, k[:, t, :])',
     'alpha = np.einsum("cij,cj->ci", A, u[:, t, 0, :])'),
    ("alpha always unit-normalised", "alpha / np.maximum(anorm, 1.0)[:, None]",
     "alpha / anorm[:, None]"),
    ("alpha never normalised", "alpha / np.maximum(anorm, 1.0)[:, None]", "alpha"),
    ("state update transposed", "S = S + v[:, t, :, None] * alpha_hat[:, None, :]",
     "S = S + v[:, t, None, :] * alpha_hat[:, :, None]"),
    ("cap scale inverted", "scale = np.where(over, s_cap / np.where(over, fn, 1.0), 1.0)",
     "scale = np.where(over, np.where(over, fn, 1.0) / s_cap, 1.0)"),
    ("cap test non-strict and on the square", "over = fn > s_cap", "over = fn * fn > s_cap"),
    ("normaliser lags one token", "n = n + k[:, t, :]\n        den = np.einsum(\"ci,ci->c\", n, q[:, t, :]) + den_eps",
     "den = np.einsum(\"ci,ci->c\", n, q[:, t, :]) + den_eps\n        n = n + k[:, t, :]"),
    ("readout denominator without its epsilon", "q[:, t, :]) + den_eps", "q[:, t, :]) + 0.0"),
    ("readout with the transposed state", 'o[:, t, :] = np.einsum("cij,cj->ci", S, q[:, t, :])',
     'o[:, t, :] = np.einsum("cji,cj->ci", S, q[:, t, :])'),
    ("readout before the update of S",
     "            S = S + v[:, t, :, None] * alpha_hat[:, None, :]\n",
     "            o_prev = np.einsum(\"cij,cj->ci\", S, q[:, t, :])\n"
     "            S = S + v[:, t, :, None] * alpha_hat[:, None, :]\n"),
    ("alpha from the inverse before the token's updates",
     "        for i in range(r):\n", "        A_prev = A\n        for i in range(r):\n"),
    ("nudge applied after alpha",
     "        if nudge_period > 0 and tau % nudge_period == 0:\n            A = A + eps * eye\n", ""),
    ("cap applied after the readout",
     "        if cap_on:\n            over = fn > s_cap", "        if False:\n            over = fn > s_cap"),
    ("first cap step off by one", "first_cap = np.where(over & (first_cap < 0), t, first_cap)",
     "first_cap = np.where(over & (first_cap < 0), t + 1, first_cap)"),
    ("first cap step records the latest fire", "first_cap = np.where(over & (first_cap < 0), t, first_cap)",
     "first_cap = np.where(over, t, first_cap)"),
    ("bfloat16 widened through float16",
     "        if x.dtype in (torch.bfloat16, torch.float16):\n            x = x.to(torch.float32)",
     "        if x.dtype in (torch.bfloat16, torch.float16):\n            x = x.to(torch.float16).to(torch.float32)"),
    ("float32 tensors rounded through bfloat16",
     "        if x.dtype in (torch.bfloat16, torch.float16):\n            x = x.to(torch.float32)",
     "        if x.dtype in (torch.bfloat16, torch.float16, torch.float32):\n"
     "            x = x.to(torch.bfloat16).to(torch.float32)"),
    ("residual with the wrong sign", "resid = v[:, t, :] - np.einsum", "resid = v[:, t, :] + np.einsum"),
    ("residual predicted from the raw key", 'resid = v[:, t, :] - np.einsum("cij,cj->ci", S, khat)',
     'resid = v[:, t, :] - np.einsum("cij,cj->ci", S, k[:, t, :])'),
    ("residual key not normalised", "khat = _normalize_rows(k[:, t, :]) if normalize else k[:, t, :]",
     "khat = k[:, t, :]"),
    ("residual gate clamped instead of unit", "alpha_hat = _normalize_rows(alpha) if normalize else alpha",
     "alpha_hat = alpha / np.maximum(np.sqrt(np.einsum('ci,ci->c', alpha, alpha)), 1.0)[:, None] "
     "if normalize else alpha"),
    ("residual written along the key instead of the gate",
     "S = S + resid[:, :, None] * alpha_hat[:, None, :]", "S = S + resid[:, :, None] * khat[:, None, :]"),
    ("residual update transposed", "S = S + resid[:, :, None] * alpha_hat[:, None, :]",
     "S = S + resid[:, None, :] * alpha_hat[:, :, None]"),
    ("residual gate from the inverse before the token's updates",
     "        for i in range(r):\n", "        A_prev = A\n        for i in range(r):\n"),
    ("residual written from the initial state", "resid = v[:, t, :] - np.einsum(\"cij,cj->ci\", S, khat)",
     "resid = v[:, t, :] - np.einsum(\"cij,cj->ci\", S0c, khat)"),
    ("projection applies W^T", "x = rows @ W[i].T", "x = rows @ W[i]"),
    ("projection not normalised", "out[:, i, :] = x / np.maximum(nrm, 1e-12)[:, None]",
     "out[:, i, :] = x"),
]
# The "readout before the update" mutant needs its value used; patch the store too.
_EXTRA = {
    "alpha from the inverse before the token's updates": [
        ('alpha = np.einsum("cij,cj->ci", A, k[:, t, :])', 'alpha = np.einsum("cij,cj->ci", A_prev, k[:, t, :])')],
    "nudge applied after alpha": [
        ("            alpha_hat = alpha / np.maximum(anorm, 1.0)[:, None]\n",
         "            alpha_hat = alpha / np.maximum(anorm, 1.0)[:, None]\n"
         "            if nudge_period > 0 and tau % nudge_period == 0:\n                A = A + eps * eye\n")],
    "cap applied after the readout": [
        ("        o[:, t, :] = np.einsum(\"cij,cj->ci\", S, q[:, t, :]) / den[:, None]\n",
         "        o[:, t, :] = np.einsum(\"cij,cj->ci\", S, q[:, t, :]) / den[:, None]\n"
         "        if cap_on:\n"
         "            over = fn > s_cap\n"
         "            scale = np.where(over, s_cap / np.where(over, fn, 1.0), 1.0)\n"
         "            S = S * scale[:, None, None]\n"
         "            first_cap = np.where(over & (first_cap < 0), t, first_cap)\n"
         "            capf += over\n"
         "            fn = np.where(over, s_cap, fn)\n")],
    "residual gate from the inverse before the token's updates": [
        ('alpha = np.einsum("cij,cj->ci", A, khat)', 'alpha = np.einsum("cij,cj->ci", A_prev, khat)')],
    "residual written from the initial state": [
        ("    guard = np.zeros(C, dtype=np.int64)\n", "    S0c = S.copy()\n    guard = np.zeros(C, dtype=np.int64)\n")],
    "readout before the update of S": [
        ('o[:, t, :] = np.einsum("cij,cj->ci", S, q[:, t, :]) / den[:, None]',
         'o[:, t, :] = o_prev / den[:, None]')],
}

PINS = [
    ("test_hand_worked_fixture", {"name": "hand_d2_plain.txt"}),
    ("test_as_f64_widens_torch_tensors_exactly", {}),
    ("test_first_cap_step_closed_form", {}),
    ("test_hand_worked_fixture", {"name": "hand_d2_guard_nudge_cap.txt"}),
    ("test_inverse_tracking_matches_direct_inverse", {"spd_start": True}),
    ("test_alpha_uses_post_update_inverse", {}),
    ("test_rank_r_matches_woodbury", {"r": 2}),
    ("test_guard_silent_on_spd_inputs", {}),
    ("test_guard_fire_skips_update_and_injects_eps", {}),
    ("test_indefinite_start_divides_by_signed_delta", {}),
    ("test_nudge_piecewise_closed_form", {"t0": 3}),
    ("test_spectrum_invariants", {}),
    ("test_alpha_clamp_invariant", {}),
    ("test_cap_bounds_state_and_forced_first_step", {}),
    ("test_zero_u_is_causal_linear_attention", {"kscale": 1.0}),
    ("test_linearity_in_values_and_initial_state", {}),
    ("test_resume_equivalence", {}),
    ("test_project_u_closed_forms", {}),
    ("test_residual_unnormalised_is_recursive_least_squares", {}),
    ("test_residual_orthogonal_keys_closed_form", {"with_u": True}),
    ("test_residual_first_step_gate_is_unit_and_nudged", {}),
    ("test_residual_invariants_linearity_resume_cap", {}),
]


def _load_mutant(desc, old, new):
    with open(ORACLE_SRC) as f:
        src = f.read()
    edits = [(old, new)] + _EXTRA.get(desc, [])
    for o, n in edits:
        assert src.count(o) == 1, f"mutation anchor not unique for {desc!r}: {o!r}"
        src = src.replace(o, n)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, f"<mutant: {desc}>", "exec"), mod.__dict__)
    return mod


def test_pins_pass_on_the_oracle():
    for name, kw in PINS:
        getattr(pins, name)(**kw)


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(desc, old, new, monkeypatch):
    mod = _load_mutant(desc, old, new)
    monkeypatch.setattr(pins, "oracle_scan", mod.oracle_scan)
    monkeypatch.setattr(pins, "oracle_project_u", mod.oracle_project_u)
    monkeypatch.setattr(pins, "as_f64", mod.as_f64)
    caught = []
    for name, kw in PINS:
        try:
            getattr(pins, name)(**kw)
        except Exception as e:  # an assertion, or the mutant crashing outright
            caught.append(f"{name}{kw}: {type(e).__name__}")
    assert caught, f"no pin catches the planted mistake: {desc}"

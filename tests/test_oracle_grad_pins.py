"""Pins of the gradient oracle (oracle_scan_grad) against facts other than itself.

* Its forward values equal the float64 NumPy oracle's (the transcription of
  the recurrence is the same recurrence), with the guard, the nudge, the
  clamp and the cap all active.
* Its gradients equal central finite differences of the NumPy oracle
  (``oracle_scan``) itself, along random directions, for every input.
* At u = 0, A0 = I, no nudge, no cap and |k| <= 1 the scan is causal linear
  attention, whose gradient with respect to v has a closed form.
* A guard fire skips its rank-1 step, so that direction gets no gradient.
Planted mistakes in the transcription are caught (last test).
"""
import types

import numpy as np
import pytest

from oracle.vla_oracle import oracle_scan
from oracle import vla_oracle_grad
from oracle.vla_oracle_grad import oracle_scan_grad

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _inputs(C, T, d, r, seed, kscale=1.0):
    g = np.random.default_rng(seed)
    elu1 = lambda x: np.where(x > 0, x, np.expm1(x)) + 1.0
    q = elu1(g.standard_normal((C, T, d)))
    k = kscale * elu1(g.standard_normal((C, T, d)))
    v = g.standard_normal((C, T, d))
    u = g.standard_normal((C, T, r, d))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    X = g.standard_normal((C, d, d)) / d
    A0 = 0.6 * np.eye(d) + X @ X.transpose(0, 2, 1)
    S0 = g.standard_normal((C, d, d))
    n0 = g.random((C, d))
    cots = dict(g_o=g.standard_normal((C, T, d)), g_A=g.standard_normal((C, d, d)),
                g_S=g.standard_normal((C, d, d)), g_n=g.standard_normal((C, d)))
    return dict(q=q, k=k, v=v, u=u, A0=A0, S0=S0, n0=n0), cots


KW = dict(nudge_period=3, s_cap=4.0, t0=1)


def _loss(ins, cots, **kw):
    res = oracle_scan(ins["q"], ins["k"], ins["v"], ins["u"], ins["A0"], ins["S0"], ins["n0"], **kw)
    return ((res["o"] * cots["g_o"]).sum() + (res["A"] * cots["g_A"]).sum() + (res["S"] * cots["g_S"]).sum()
            + (res["n"] * cots["g_n"]).sum()), res


def test_forward_values_equal_the_numpy_oracle():
    ins, cots = _inputs(3, 9, 5, 2, seed=1)
    _, ref = _loss(ins, cots, **KW)
    assert ref["cap_fires"].min() > 0
    got = oracle_scan_grad(**ins, **cots, **KW)
    for name in ("o", "A", "S", "n"):
        np.testing.assert_allclose(got[name], ref[name], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("name", ["q", "k", "v", "u", "A0", "S0", "n0"])
def test_gradients_equal_central_differences(name):
    ins, cots = _inputs(2, 7, 4, 2, seed=2)
    grads = oracle_scan_grad(**ins, **cots, **KW)
    g = np.random.default_rng(3)
    h = 1e-6
    for _ in range(3):
        dirn = g.standard_normal(ins[name].shape)
        plus = dict(ins)
        minus = dict(ins)
        plus[name] = ins[name] + h * dirn
        minus[name] = ins[name] - h * dirn
        lp, rp = _loss(plus, cots, **KW)
        lm, rm = _loss(minus, cots, **KW)
        # the cap and guard decisions are the same on both sides (smooth region)
        assert (rp["cap_fires"] == rm["cap_fires"]).all()
        fd = (lp - lm) / (2 * h)
        an = float((grads[name] * dirn).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_linear_attention_closed_form_for_values():
    C, T, d = 2, 12, 4
    ins, cots = _inputs(C, T, d, 1, seed=4, kscale=0.1)
    ins["u"] = np.zeros_like(ins["u"])
    ins["A0"] = np.broadcast_to(np.eye(d), (C, d, d)).copy()
    ins["S0"] = np.zeros((C, d, d))
    ins["n0"] = np.zeros((C, d))
    assert (np.linalg.norm(ins["k"], axis=-1) <= 1).all()
    grads = oracle_scan_grad(**ins, g_o=cots["g_o"])
    q, k, go = ins["q"], ins["k"], cots["g_o"]
    # o_t = sum_{s<=t} v_s (k_s.q_t) / den_t,  den_t = sum_{s<=t} k_s.q_t + 1e-6
    kq = np.einsum("csi,cti->cts", k, q)
    den = np.cumsum(kq * np.tri(T)[None], axis=2)[:, np.arange(T), np.arange(T)] + 1e-6
    w = kq * np.tri(T)[None] / den[:, :, None]            # w[c, t, s]
    gv = np.einsum("cts,cti->csi", w, go)
    np.testing.assert_allclose(grads["v"], gv, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(grads["u"], 0.0)


def test_guard_fire_gives_no_gradient_to_its_direction():
    d, T = 4, 3
    ins, cots = _inputs(1, T, d, 1, seed=5)
    e = np.eye(d)[1]
    ins["A0"] = (np.eye(d) - 2 * np.outer(e, e))[None]
    ins["u"][0, 0, 0] = e
    res = oracle_scan(ins["q"], ins["k"], ins["v"], ins["u"], ins["A0"])
    assert res["guard_fires"][0] == 1
    grads = oracle_scan_grad(ins["q"], ins["k"], ins["v"], ins["u"], ins["A0"], g_o=cots["g_o"], g_S=cots["g_S"])
    np.testing.assert_array_equal(grads["u"][0, 0], 0.0)
    assert np.abs(grads["u"][0, 1:]).max() > 0


GRAD_MUTANTS = [
    ("nudge before the rank-1 steps", "        tau = t0 + t + 1\n        if nudge_period > 0 and tau % nudge_period == 0:\n            A = A + eps * eye\n", ""),
    ("alpha not clamped", "alpha_hat = alpha / torch.clamp(anorm, min=1.0)[:, None]", "alpha_hat = alpha"),
    ("state update transposed", "S = S + v[:, t, :, None] * alpha_hat[:, None, :]",
     "S = S + v[:, t, None, :] * alpha_hat[:, :, None]"),
    ("readout before the normaliser update", "        n = n + k[:, t, :]\n        den =",
     "        den_n = n\n        n = n + k[:, t, :]\n        den ="),
    ("cap test non-strict on the square", "over = fn > s_cap", "over = fn * fn > s_cap"),
]


@pytest.mark.parametrize("desc,old,new", GRAD_MUTANTS, ids=[m[0] for m in GRAD_MUTANTS])
def test_planted_mistake_in_the_transcription_is_caught(desc, old, new):
    src = open(vla_oracle_grad.__file__).read()
    assert src.count(old) == 1, desc
    src = src.replace(old, new)
    if desc == "nudge before the rank-1 steps":
        src = src.replace("        for i in range(r):   # r sequential",
                          "        tau = t0 + t + 1\n        if nudge_period > 0 and tau % nudge_period == 0:\n"
                          "            A = A + eps * eye\n        for i in range(r):   # r sequential")
    if desc == "readout before the normaliser update":
        src = src.replace("den = (n * q[:, t, :]).sum(-1) + den_eps", "den = (den_n * q[:, t, :]).sum(-1) + den_eps")
    mod = types.ModuleType("grad_mutant")
    exec(compile(src, f"<grad mutant: {desc}>", "exec"), mod.__dict__)
    caught = False
    global oracle_scan_grad
    saved = oracle_scan_grad
    oracle_scan_grad = mod.oracle_scan_grad
    try:
        for pin in (test_forward_values_equal_the_numpy_oracle, test_linear_attention_closed_form_for_values):
            try:
                pin()
            except AssertionError:
                caught = True
        if not caught:
            for name in ("q", "v", "A0"):
                try:
                    test_gradients_equal_central_differences(name)
                except AssertionError:
                    caught = True
    finally:
        oracle_scan_grad = saved
    assert caught, desc

"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: hand-worked
closed-form values, a direct matrix inverse, the Woodbury identity, textbook
causal linear attention, invariants, or a 50-digit brute force.  Together they
are chosen so that a plausible slip in the oracle (a dropped term, a wrong sign
or index, a transposed operand, a step taken at the wrong time) fails at least
one of them; ``test_planted_mistakes_are_caught`` checks that claim directly
by planting such slips in a copy of the oracle.
"""
import math

import numpy as np
import pytest

from oracle.vla_oracle import as_f64, oracle_project_u, oracle_scan
from tests import golden_io

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_inputs(C, T, d, r, seed=0, kscale=1.0):
    g = _rng(seed)
    elu1 = lambda x: np.where(x > 0, x, np.expm1(x)) + 1.0
    q = elu1(g.standard_normal((C, T, d)))
    k = kscale * elu1(g.standard_normal((C, T, d)))
    v = g.standard_normal((C, T, d))
    u = _unit(g.standard_normal((C, T, r, d)))
    return q, k, v, u


def _spd(d, seed):
    g = _rng(seed)
    X = g.standard_normal((d, d))
    return X @ X.T / d + 0.5 * np.eye(d)


# --------------------------------------------------------------------------
# Hand-worked fixtures ("Mathematical Primitives" sections 2, 4, 5; README v3
# notes item 5).  Values are exact expressions worked out by hand.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["hand_d2_plain.txt", "hand_d2_guard_nudge_cap.txt"])
def test_hand_worked_fixture(name):
    g = golden_io.load(name)
    d, r = int(g["d"]), int(g["r"])
    T = len(g["k"]) // d
    res = oracle_scan(
        np.array(g["q"]).reshape(1, T, d), np.array(g["k"]).reshape(1, T, d),
        np.array(g["v"]).reshape(1, T, d), np.array(g["u"]).reshape(1, T, r, d),
        A0=np.array(g["A0"]).reshape(1, d, d), eps=g["eps"],
        nudge_period=int(g["nudge_period"]), s_cap=g["s_cap"])
    np.testing.assert_allclose(res["o"].ravel(), g["expect_o"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(res["A"].ravel(), g["expect_A"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(res["S"].ravel(), g["expect_S"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(res["n"].ravel(), g["expect_n"], rtol=0, atol=0)
    assert int(res["guard_fires"][0]) == int(g["expect_guard_fires"])
    assert int(res["cap_fires"][0]) == int(g["expect_cap_fires"])
    assert int(res["first_cap_step"][0]) == int(g["expect_first_cap_step"])


# --------------------------------------------------------------------------
# Exact widening of stored inputs.  The workloads store q, k, v, u as float32
# or bfloat16; the oracle must see exactly the stored values.  The expected
# value of every encoding is decoded here from its bits (sign, exponent,
# significand) with exact power-of-two scaling, independently of any float
# conversion routine.
# --------------------------------------------------------------------------
def _decode_bits(bits, exp_bits, man_bits):
    bits = bits.astype(np.int64)
    bias = (1 << (exp_bits - 1)) - 1
    sign = np.where((bits >> (exp_bits + man_bits)) & 1, -1.0, 1.0)
    e = (bits >> man_bits) & ((1 << exp_bits) - 1)
    m = (bits & ((1 << man_bits) - 1)).astype(np.float64)
    normal = np.ldexp(1.0 + m / (1 << man_bits), (e - bias).astype(np.int32))
    sub = np.ldexp(m, np.int32(1 - bias - man_bits))
    val = sign * np.where(e == 0, sub, normal)
    special = e == (1 << exp_bits) - 1
    val = np.where(special & (m == 0), sign * np.inf, val)
    return np.where(special & (m != 0), np.nan, val)


def test_as_f64_widens_torch_tensors_exactly():
    import torch

    with np.errstate(invalid="ignore"):   # signalling NaN encodings warn when widened
        _as_f64_checks(torch)


def _as_f64_checks(torch):

    # bfloat16 and float16: every one of the 65536 encodings, including the
    # exponent extremes, subnormals, signed zeros, infinities and NaNs.
    every16 = np.arange(1 << 16, dtype=np.int64)
    as_i16 = torch.from_numpy(every16.astype(np.uint16).view(np.int16))
    for dt, e_bits, m_bits in ((torch.bfloat16, 8, 7), (torch.float16, 5, 10)):
        got = as_f64(as_i16.view(dt))
        want = _decode_bits(every16, e_bits, m_bits)
        assert got.dtype == np.float64 and got.shape == want.shape
        assert np.array_equal(np.isnan(got), np.isnan(want)), dt
        ok = ~np.isnan(want)
        assert np.array_equal(got[ok], want[ok]), dt
        assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok])), dt
    # float32: the edge encodings plus a random sample of all others.
    g = _rng(40)
    edges = np.array([0, 1, 2, 0x007FFFFF, 0x00800000, 0x00800001, 0x3F800000, 0x3F800001, 0x7F7FFFFF,
                      0x7F800000, 0x7FC00000, 0x80000000, 0x80000001, 0xFF7FFFFF, 0xFF800000], dtype=np.int64)
    bits32 = np.concatenate([edges, g.integers(0, 1 << 32, 200_000, dtype=np.int64)])
    t32 = torch.from_numpy(bits32.astype(np.uint32).view(np.int32)).view(torch.float32)
    got, want = as_f64(t32), _decode_bits(bits32, 8, 23)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    # a view with a gradient, laid out non-contiguously, keeps shape and values
    base = torch.arange(24, dtype=torch.float32, requires_grad=True).reshape(4, 6)
    view = base.t()[1:5].to(torch.bfloat16)
    np.testing.assert_array_equal(as_f64(view), np.arange(24.0).reshape(4, 6).T[1:5])
    # the scan itself sees the stored bfloat16 values: one token, d = 1
    # (u = 0 so A = 1; alpha = k; S = v min(1, 1/k) k; o = S q / (k q + eps))
    kq = torch.tensor([[[3.0]]], dtype=torch.float32).to(torch.bfloat16)
    vv = torch.tensor([[[1.0 / 3.0]]], dtype=torch.float32).to(torch.bfloat16)
    res = oracle_scan(kq, kq, vv, torch.zeros(1, 1, 1, 1, dtype=torch.bfloat16))
    v_stored = _decode_bits(np.array([int(vv.view(torch.int16).item()) & 0xFFFF]), 8, 7)[0]
    assert v_stored != 1.0 / 3.0
    np.testing.assert_allclose(res["S"][0, 0, 0], v_stored, rtol=1e-15)


# --------------------------------------------------------------------------
# First cap step ("Mathematical Primitives", section 5, dynamic
# renormalisation; strict test, checked after every state update).  With
# u = 0, A0 = I, no nudge and k_t = e1 (so alpha_hat = e1), v_t = c e1 makes
# S_t = t c e1 e1^T (t 1-based) until the first fire, which therefore comes
# at the smallest 0-based index f with (f + 1) c > cap; after it S sits at
# the cap and every later token fires again.
# --------------------------------------------------------------------------
def test_first_cap_step_closed_form():
    d, T = 3, 12
    rates = np.array([1.0, 2.0, 0.5, 4.0, 0.25])
    C = len(rates)
    e1 = np.eye(d)[0]
    k = np.broadcast_to(e1, (C, T, d)).copy()
    v = rates[:, None, None] * k
    q = np.broadcast_to(np.array([1.0, 0.5, 0.25]), (C, T, d)).copy()
    u = np.zeros((C, T, 1, d))
    for cap in (0.1, 1.0, 2.0, 5.5, 6.0, 7.5, 100.0):
        res = oracle_scan(q, k, v, u, s_cap=cap)
        for c, rate in enumerate(rates):
            f = next((i for i in range(T) if (i + 1) * rate > cap), -1)
            assert int(res["first_cap_step"][c]) == f, (cap, rate)
            assert int(res["cap_fires"][c]) == (T - f if f >= 0 else 0), (cap, rate)
    # a chain that never reaches the cap reports -1, beside one that does
    res = oracle_scan(q[:2], k[:2], v[:2] * np.array([1.0, 0.0])[:, None, None], u[:2], s_cap=3.0)
    assert list(res["first_cap_step"]) == [3, -1]


# --------------------------------------------------------------------------
# Sherman-Morrison tracking equals the direct inverse of the explicitly built
# penalty matrix M_t = A0^{-1} + sum u u^T ("Mathematical Primitives",
# section 2, theoretical derivation), and alpha = A_t k_t (section 4).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("spd_start", [False, True])
def test_inverse_tracking_matches_direct_inverse(spd_start):
    d, T = 8, 40
    q, k, v, u = _rand_inputs(1, T, d, 1, seed=1)
    A0 = _spd(d, 2) if spd_start else np.eye(d)
    M = np.linalg.inv(A0)
    for t in range(T):
        M = M + np.outer(u[0, t, 0], u[0, t, 0])
        if t in (0, 1, 7, 20, T - 1):
            res = oracle_scan(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], u[:, :t + 1], A0=A0[None])
            np.testing.assert_allclose(res["A"][0] @ M, np.eye(d), atol=1e-11)
            np.testing.assert_allclose(res["A"][0], np.linalg.inv(M), rtol=1e-10, atol=1e-12)


def test_alpha_uses_post_update_inverse():
    """alpha_t = A_t k_t with A_t after token t's update, read out through S."""
    d, T = 6, 6
    q, k, v, u = _rand_inputs(1, T, d, 1, seed=3, kscale=0.05)
    vv = np.zeros_like(v)
    for t in range(T):
        vv[0, t, t] = 1.0   # v_t = e_t, so row t of S_T is alpha_hat_t
    res = oracle_scan(q, k, vv, u)
    M = np.eye(d)
    for t in range(T):
        M = M + np.outer(u[0, t, 0], u[0, t, 0])
        alpha = np.linalg.solve(M, k[0, t])
        ahat = alpha / max(np.linalg.norm(alpha), 1.0)
        np.testing.assert_allclose(res["S"][0, t], ahat, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# Rank r as r sequential rank-1 updates equals the closed-form Woodbury
# inverse ("Mathematical Primitives", section 3).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("r", [2, 4])
def test_rank_r_matches_woodbury(r):
    d = 8
    q, k, v, u = _rand_inputs(1, 3, d, r, seed=4)
    A0 = _spd(d, 5)
    A = A0.copy()
    for t in range(3):
        U = u[0, t].T                                      # [d, r]
        A = A - A @ U @ np.linalg.solve(np.eye(r) + U.T @ A @ U, U.T @ A)
        res = oracle_scan(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], u[:, :t + 1], A0=A0[None])
        np.testing.assert_allclose(res["A"][0], A, rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------
# The guard never fires on SPD state: delta = 1 + u^T A u >= 1 for A >= 0.
# --------------------------------------------------------------------------
def test_guard_silent_on_spd_inputs():
    q, k, v, u = _rand_inputs(16, 300, 8, 3, seed=6)
    res = oracle_scan(q, k, v, u, nudge_period=16, s_cap=5.0)
    assert res["guard_fires"].sum() == 0
    w, _ = np.linalg.eigh(res["A"])
    assert (w > 0).all()


def test_guard_fire_skips_update_and_injects_eps():
    """Householder start A0 = I - 2 u u^T makes delta exactly 0 on the first step."""
    d = 4
    g = _rng(7)
    u1 = np.zeros(d)
    u1[2] = 1.0
    A0 = np.eye(d) - 2.0 * np.outer(u1, u1)
    k = np.abs(g.standard_normal((1, 1, d))) + 0.5
    q = np.abs(g.standard_normal((1, 1, d))) + 0.5
    v = g.standard_normal((1, 1, d))
    for eps in (1e-6, 0.25):
        res = oracle_scan(q, k, v, u1.reshape(1, 1, 1, d), A0=A0[None], eps=eps)
        A1 = A0 + eps * np.eye(d)
        np.testing.assert_allclose(res["A"][0], A1, rtol=0, atol=1e-15)
        alpha = A1 @ k[0, 0]
        ahat = alpha / max(np.linalg.norm(alpha), 1.0)
        S1 = np.outer(v[0, 0], ahat)
        np.testing.assert_allclose(res["S"][0], S1, rtol=1e-14, atol=1e-15)
        o1 = S1 @ q[0, 0] / (k[0, 0] @ q[0, 0] + 1e-6)
        np.testing.assert_allclose(res["o"][0, 0], o1, rtol=1e-14, atol=1e-15)
        assert res["guard_fires"][0] == 1


def test_indefinite_start_divides_by_signed_delta():
    """A0 = diag(-2, 1, ...) and u = e1 give delta = -1, well outside the guard:
    the update divides by the signed delta and still equals the direct inverse
    of A0^{-1} + u u^T = diag(1/2, 1, ...), i.e. diag(2, 1, ...)."""
    d = 4
    g = _rng(21)
    A0 = np.eye(d)
    A0[0, 0] = -2.0
    u1 = np.zeros((1, 1, 1, d))
    u1[0, 0, 0, 0] = 1.0
    k = np.abs(g.standard_normal((1, 1, d))) + 0.5
    q = np.abs(g.standard_normal((1, 1, d))) + 0.5
    v = g.standard_normal((1, 1, d))
    res = oracle_scan(q, k, v, u1, A0=A0[None])
    A1 = np.eye(d)
    A1[0, 0] = 2.0
    np.testing.assert_allclose(res["A"][0], A1, rtol=1e-15, atol=1e-15)
    assert res["guard_fires"][0] == 0


# --------------------------------------------------------------------------
# Periodic nudge: between nudges A is the inverse of the accumulated penalty;
# at every multiple of the period eps*I is added after the rank-1 update and
# before alpha ("Mathematical Primitives", section 2, periodic spectrum
# stabilisation).  A large eps makes every term visible.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("t0", [0, 3])
def test_nudge_piecewise_closed_form(t0):
    d, T, P, eps = 5, 13, 4, 0.05
    q, k, v, u = _rand_inputs(1, T, d, 1, seed=8, kscale=0.1)
    res_all = []
    A = np.eye(d)
    for t in range(T):
        A = np.linalg.inv(np.linalg.inv(A) + np.outer(u[0, t, 0], u[0, t, 0]))
        if (t0 + t + 1) % P == 0:
            A = A + eps * np.eye(d)
        res_all.append(A.copy())
    res = oracle_scan(q, k, v, u, eps=eps, nudge_period=P, t0=t0)
    np.testing.assert_allclose(res["A"][0], res_all[-1], rtol=1e-11, atol=1e-13)
    # alpha at a nudge step sees the nudged inverse: read it back through S.
    tn = next(t for t in range(T) if (t0 + t + 1) % P == 0)
    vv = np.zeros_like(v)
    vv[0, tn, 0] = 1.0
    res1 = oracle_scan(q[:, :tn + 1], k[:, :tn + 1], vv[:, :tn + 1], u[:, :tn + 1],
                       eps=eps, nudge_period=P, t0=t0)
    alpha = res_all[tn] @ k[0, tn]
    ahat = alpha / max(np.linalg.norm(alpha), 1.0)
    np.testing.assert_allclose(res1["S"][0, 0], ahat, rtol=1e-11, atol=1e-14)


def test_spectrum_invariants():
    """A0 = I, no nudge: 0 < lambda(A_t) <= 1, A_t <= A_{t-1} (Loewner), tr A non-increasing.
    With nudges: lambda_max <= 1 + (number of nudges) * eps."""
    d, T = 6, 48
    q, k, v, u = _rand_inputs(1, T, d, 2, seed=9)
    prev = np.eye(d)
    for t in range(1, T + 1, 4):
        A = oracle_scan(q[:, :t], k[:, :t], v[:, :t], u[:, :t])["A"][0]
        w = np.linalg.eigvalsh(A)
        assert w.min() > 0 and w.max() <= 1 + 1e-12
        assert np.linalg.eigvalsh(prev - A).min() >= -1e-12
        assert np.trace(A) <= np.trace(prev) + 1e-12
        prev = A
    eps, P = 1e-3, 5
    A = oracle_scan(q, k, v, u, eps=eps, nudge_period=P)["A"][0]
    assert np.linalg.eigvalsh(A).max() <= 1 + (T // P) * eps + 1e-12


# --------------------------------------------------------------------------
# alpha_hat = alpha / max(|alpha|, 1): |alpha_hat| <= 1, with equality exactly
# when |alpha| >= 1 (README v3 notes item 4; reading of the clamp).
# --------------------------------------------------------------------------
def test_alpha_clamp_invariant():
    d, T = 8, 8
    for kscale, expect_unit in ((3.0, True), (0.02, False)):
        q, k, v, u = _rand_inputs(1, T, d, 1, seed=10, kscale=kscale)
        vv = np.zeros_like(v)
        for t in range(T):
            vv[0, t, t] = 1.0
        S = oracle_scan(q, k, vv, u)["S"][0]
        norms = np.linalg.norm(S, axis=1)
        M = np.eye(d)
        for t in range(T):
            M = M + np.outer(u[0, t, 0], u[0, t, 0])
            an = np.linalg.norm(np.linalg.solve(M, k[0, t]))
            assert (an >= 1) == expect_unit
            if expect_unit:
                assert abs(norms[t] - 1.0) < 1e-13
            else:
                assert abs(norms[t] - an) < 1e-15 and norms[t] < 1


# --------------------------------------------------------------------------
# Frobenius cap ("Mathematical Primitives", section 5, dynamic renormalisation).
# --------------------------------------------------------------------------
def test_cap_bounds_state_and_forced_first_step():
    d, T = 8, 200
    q, k, v, u = _rand_inputs(4, T, d, 1, seed=11)
    cap = 3.0
    res = oracle_scan(q, k, v, u, s_cap=cap)
    assert (res["max_s_norm"] <= cap * (1 + 1e-12)).all()
    assert (np.linalg.norm(res["S"], axis=(1, 2)) <= cap * (1 + 1e-12)).all()
    assert (res["cap_fires"] > 0).all()
    # forced: cap = 1 at t = 1
    one = oracle_scan(q[:, :1], k[:, :1], v[:, :1], u[:, :1], s_cap=1.0)
    for c in range(4):
        M = np.eye(d) + np.outer(u[c, 0, 0], u[c, 0, 0])
        alpha = np.linalg.solve(M, k[c, 0])
        ahat = alpha / max(np.linalg.norm(alpha), 1.0)
        scale = min(1.0, 1.0 / (np.linalg.norm(v[c, 0]) * np.linalg.norm(ahat)))
        S1 = np.outer(v[c, 0], ahat) * scale
        np.testing.assert_allclose(one["S"][c], S1, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(one["o"][c, 0], S1 @ q[c, 0] / (k[c, 0] @ q[c, 0] + 1e-6),
                                   rtol=1e-13, atol=1e-15)
    # a cap above the uncapped maximum never fires; one just below it fires
    base = oracle_scan(q, k, v, u)
    m = base["max_s_norm"]
    assert (m > 1.5).all()
    hi = oracle_scan(q, k, v, u, s_cap=float(m.max()) * 1.001)
    assert hi["cap_fires"].sum() == 0
    np.testing.assert_array_equal(hi["o"], base["o"])
    lo = oracle_scan(q, k, v, u, s_cap=float(m.min()) * 0.999)
    assert (lo["cap_fires"] >= 1).all()
    np.testing.assert_allclose(lo["max_s_norm"], float(m.min()) * 0.999, rtol=1e-13)
    # cap disabled by None, 0 and inf alike
    for off in (None, 0.0, -1.0, math.inf):
        np.testing.assert_array_equal(oracle_scan(q, k, v, u, s_cap=off)["o"], base["o"])


# --------------------------------------------------------------------------
# u = 0 leaves A = I, and the scan becomes causal linear attention, computed
# here through the O(T^2) masked attention-matrix form.  When every |k| <= 1 it
# is exactly textbook causal linear attention.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kscale", [1.0, 0.05])
def test_zero_u_is_causal_linear_attention(kscale):
    C, T, d = 3, 50, 8
    q, k, v, _ = _rand_inputs(C, T, d, 1, seed=12, kscale=kscale)
    u = np.zeros((C, T, 1, d))
    res = oracle_scan(q, k, v, u)
    mask = np.tril(np.ones((T, T)))
    for c in range(C):
        khat = k[c] / np.maximum(np.linalg.norm(k[c], axis=1), 1.0)[:, None]
        num = (mask * (q[c] @ khat.T)) @ v[c]                 # sum_s (khat_s . q_t) v_s
        den = (mask * (q[c] @ k[c].T)).sum(axis=1) + 1e-6     # sum_s k_s . q_t
        np.testing.assert_allclose(res["o"][c], num / den[:, None], rtol=1e-11, atol=1e-13)
        if kscale < 1:
            assert (np.linalg.norm(k[c], axis=1) <= 1).all()
            lin = (mask * (q[c] @ k[c].T)) @ v[c] / den[:, None]
            np.testing.assert_allclose(res["o"][c], lin, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(res["A"], np.broadcast_to(np.eye(d), (C, d, d)), atol=0)


# --------------------------------------------------------------------------
# With the cap off, (o, S_T) is linear in (v, S0), and A_T does not depend on v.
# --------------------------------------------------------------------------
def test_linearity_in_values_and_initial_state():
    C, T, d = 2, 30, 8
    q, k, v1, u = _rand_inputs(C, T, d, 1, seed=13)
    g = _rng(14)
    v2 = g.standard_normal(v1.shape)
    S1 = g.standard_normal((C, d, d))
    S2 = g.standard_normal((C, d, d))
    a = oracle_scan(q, k, v1, u, S0=S1)
    b = oracle_scan(q, k, v2, u, S0=S2)
    c = oracle_scan(q, k, v1 - 2.5 * v2, u, S0=S1 - 2.5 * S2)
    np.testing.assert_allclose(c["o"], a["o"] - 2.5 * b["o"], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(c["S"], a["S"] - 2.5 * b["S"], rtol=1e-10, atol=1e-10)
    np.testing.assert_array_equal(a["A"], b["A"])


# --------------------------------------------------------------------------
# Resume: scan(0..T) equals scan(0..T1) followed by scan(T1..T) with the state
# carried and t0 = T1 (the nudge phase follows the global token index).
# --------------------------------------------------------------------------
def test_resume_equivalence():
    C, T, T1, d = 3, 70, 29, 8
    q, k, v, u = _rand_inputs(C, T, d, 2, seed=15)
    kw = dict(nudge_period=8, s_cap=4.0, eps=1e-3)
    full = oracle_scan(q, k, v, u, **kw)
    a = oracle_scan(q[:, :T1], k[:, :T1], v[:, :T1], u[:, :T1], **kw)
    b = oracle_scan(q[:, T1:], k[:, T1:], v[:, T1:], u[:, T1:], A0=a["A"], S0=a["S"], n0=a["n"],
                    t0=T1, **kw)
    np.testing.assert_allclose(np.concatenate([a["o"], b["o"]], axis=1), full["o"], rtol=1e-12, atol=1e-14)
    for key in ("A", "S", "n"):
        np.testing.assert_allclose(b[key], full[key], rtol=1e-12, atol=1e-14)
    assert ((a["cap_fires"] + b["cap_fires"]) == full["cap_fires"]).all()


def test_empty_sequence_passes_state_through():
    d = 4
    g = _rng(16)
    A0, S0, n0 = _spd(d, 17)[None], g.standard_normal((1, d, d)), g.standard_normal((1, d))
    e = np.zeros((1, 0, d))
    res = oracle_scan(e, e, e, np.zeros((1, 0, 2, d)), A0=A0, S0=S0, n0=n0)
    assert res["o"].shape == (1, 0, d)
    np.testing.assert_array_equal(res["A"], A0)
    np.testing.assert_array_equal(res["S"], S0)
    np.testing.assert_array_equal(res["n"], n0)


def test_nonfinite_flag():
    q, k, v, u = _rand_inputs(2, 5, 4, 1, seed=18)
    v[1, 2, 0] = np.nan
    res = oracle_scan(q, k, v, u)
    assert list(res["nonfinite"]) == [False, True]


# --------------------------------------------------------------------------
# 50-digit brute force on tiny inputs, written with mpmath matrices and the
# direct inverse of the explicitly accumulated penalty (no Sherman-Morrison),
# agrees with the fp64 oracle to 1e-12.
# --------------------------------------------------------------------------
def test_mpmath_brute_force_tiny():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    C, T, d, r = 2, 12, 4, 2
    q, k, v, u = _rand_inputs(C, T, d, r, seed=19)
    P, cap, eps = 5, 2.0, 1e-2
    res = oracle_scan(q, k, v, u, nudge_period=P, s_cap=cap, eps=eps)
    mp = mpmath.mpf
    for c in range(C):
        A = mpmath.eye(d)
        S = mpmath.zeros(d, d)
        n = mpmath.zeros(d, 1)
        for t in range(T):
            M = A ** -1
            for i in range(r):
                uu = mpmath.matrix([mp(x) for x in u[c, t, i]])
                M = M + uu * uu.T
            A = M ** -1
            if (t + 1) % P == 0:
                A = A + mp(eps) * mpmath.eye(d)
            kk = mpmath.matrix([mp(x) for x in k[c, t]])
            alpha = A * kk
            an = mpmath.sqrt(sum(x * x for x in alpha))
            ahat = alpha / max(an, mp(1))
            vv = mpmath.matrix([mp(x) for x in v[c, t]])
            S = S + vv * ahat.T
            fn = mpmath.sqrt(sum(S[i, j] ** 2 for i in range(d) for j in range(d)))
            if fn > cap:
                S = S * (mp(cap) / fn)
            n = n + kk
            qq = mpmath.matrix([mp(x) for x in q[c, t]])
            o = S * qq / ((n.T * qq)[0] + mp("1e-6"))
            np.testing.assert_allclose([float(x) for x in o], res["o"][c, t], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(np.array(A.tolist(), dtype=float), res["A"][c], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(np.array(S.tolist(), dtype=float), res["S"][c], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# Projection u = normalize(W_u k_raw) (README v3 notes item 2).
# --------------------------------------------------------------------------
def test_project_u_closed_forms():
    g = _rng(20)
    d, rows = 6, 10
    kr = g.standard_normal((rows, d))
    # identity: u = k / |k|
    u = oracle_project_u(np.eye(d)[None], kr)
    np.testing.assert_allclose(u[:, 0], kr / np.linalg.norm(kr, axis=1, keepdims=True), rtol=1e-15)
    # orientation: W k, not W^T k.  W = E_01 maps k to (k_1, 0, ...).
    W = np.zeros((1, d, d))
    W[0, 0, 1] = 1.0
    u = oracle_project_u(W, kr)
    expect = np.zeros((rows, d))
    expect[:, 0] = np.sign(kr[:, 1])
    np.testing.assert_array_equal(u[:, 0], expect)
    # several directions, unit norm, and each one parallel to its own W_i k
    W = g.standard_normal((3, d, d))
    u = oracle_project_u(W, kr)
    np.testing.assert_allclose(np.linalg.norm(u, axis=-1), 1.0, rtol=1e-15)
    for i in range(3):
        for j in range(rows):
            x = sum(W[i, :, m] * kr[j, m] for m in range(d))
            cosang = x @ u[j, i] / np.linalg.norm(x)
            assert abs(cosang - 1.0) < 1e-14
    # zero input stays zero (normalize divides by max(|x|, 1e-12))
    assert (oracle_project_u(np.zeros((1, d, d)), kr) == 0).all()
    tiny = oracle_project_u(np.eye(d)[None] * 1e-14, np.ones((1, d)))
    np.testing.assert_allclose(tiny[0, 0], np.full(d, 1e-14 / 1e-12), rtol=1e-14)


# --------------------------------------------------------------------------
# Residual (delta-rule) update ("Variational Linear Attention: Stable
# Associative Memory for Long-Context Transformers", technical summary 2.3;
# its section 5 ties the method to recursive least squares).
# --------------------------------------------------------------------------
def test_residual_unnormalised_is_recursive_least_squares():
    # With u = k and both unit normalisations dropped, the residual scan is
    # recursive least squares: S_t M_t = S0 A0^{-1} + sum_s v_s k_s^T with
    # M_t = A0^{-1} + sum_s k_s k_s^T, i.e. S_t solves the regularised
    # least-squares problem in closed form.
    C, T, d = 2, 30, 6
    q, k, v, _ = _rand_inputs(C, T, d, 1, seed=30)
    g = _rng(31)
    A0 = np.stack([_spd(d, 32), _spd(d, 33)])
    S0 = g.standard_normal((C, d, d))
    res = oracle_scan(q, k, v, k[:, :, None, :], A0=A0, S0=S0, update="residual", normalize=False)
    for c in range(C):
        M = np.linalg.inv(A0[c])
        Y = S0[c] @ M
        n = np.zeros(d)
        for t in range(T):
            M = M + np.outer(k[c, t], k[c, t])
            Y = Y + np.outer(v[c, t], k[c, t])
            n = n + k[c, t]
            St = np.linalg.solve(M.T, Y.T).T            # Y M^{-1}
            np.testing.assert_allclose(res["o"][c, t], St @ q[c, t] / (n @ q[c, t] + 1e-6),
                                       rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(res["S"][c], St, rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(res["A"][c], np.linalg.inv(M), rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("with_u", [True, False])
def test_residual_orthogonal_keys_closed_form(with_u):
    # Keys along orthonormal directions e_t with non-unit lengths c_t.  With
    # u_t = e_t (or u = 0) and A0 = I, A_t k_hat_t is a positive multiple of
    # e_t, so the unit gate is e_t itself and the update is the delta rule:
    # S_T = S0 (I - sum e e^T) + sum v e^T, each key's value recalled exactly.
    d, T = 8, 6
    g = _rng(34)
    E, _ = np.linalg.qr(g.standard_normal((d, d)))
    E = E[:, :T].T                                        # rows e_t, orthonormal
    c = g.uniform(0.4, 3.0, size=T)
    k = (c[:, None] * E)[None]
    v = g.standard_normal((1, T, d))
    q = np.abs(g.standard_normal((1, T, d))) + 0.5
    u = E[None, :, None, :] if with_u else np.zeros((1, T, 1, d))
    S0 = g.standard_normal((1, d, d))
    res = oracle_scan(q, k, v, u, S0=S0, update="residual")
    P = np.eye(d)
    Y = np.zeros((d, d))
    n = np.zeros(d)
    for t in range(T):
        P = P - np.outer(E[t], E[t])
        Y = Y + np.outer(v[0, t], E[t])
        n = n + k[0, t]
        St = S0[0] @ P + Y
        np.testing.assert_allclose(St @ E[t], v[0, t], rtol=1e-12, atol=1e-12)
        den = n @ q[0, t] + 1e-6
        np.testing.assert_allclose(res["o"][0, t] * den, St @ q[0, t], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(res["S"][0], St, rtol=1e-12, atol=1e-12)
    A_expect = np.eye(d) - 0.5 * E.T @ E if with_u else np.eye(d)
    np.testing.assert_allclose(res["A"][0], A_expect, rtol=1e-13, atol=1e-14)


def test_residual_first_step_gate_is_unit_and_nudged():
    # From S0 = 0 the first state is v alpha_hat^T with a unit gate along
    # A_1 k, where A_1 = (A0^{-1} + sum_i u_i u_i^T)^{-1} + eps I (a nudge at
    # tau = 1 with nudge_period = 1), computed here by direct inversion.
    C, d, r, eps = 3, 6, 2, 1e-2
    q, k, v, u = _rand_inputs(C, 1, d, r, seed=35)
    A0 = np.stack([_spd(d, 36 + c) for c in range(C)])
    res = oracle_scan(q, k, v, u, A0=A0, nudge_period=1, eps=eps, update="residual")
    for c in range(C):
        M = np.linalg.inv(A0[c]) + sum(np.outer(u[c, 0, i], u[c, 0, i]) for i in range(r))
        A1 = np.linalg.inv(M) + eps * np.eye(d)
        gate = A1 @ k[c, 0]
        gate = gate / np.linalg.norm(gate)
        np.testing.assert_allclose(res["S"][c], np.outer(v[c, 0], gate), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(np.linalg.norm(res["S"][c]), np.linalg.norm(v[c, 0]), rtol=1e-13)
        np.testing.assert_allclose(res["A"][c], A1, rtol=1e-12, atol=1e-14)


def test_residual_invariants_linearity_resume_cap():
    C, T, T1, d = 3, 60, 23, 8
    q, k, v1, u = _rand_inputs(C, T, d, 2, seed=37)
    g = _rng(38)
    v2 = g.standard_normal(v1.shape)
    S1, S2 = g.standard_normal((C, d, d)), g.standard_normal((C, d, d))
    kw = dict(update="residual", nudge_period=8, eps=1e-3)
    # linear in (v, S0) with the cap off; A does not depend on v
    a = oracle_scan(q, k, v1, u, S0=S1, **kw)
    b = oracle_scan(q, k, v2, u, S0=S2, **kw)
    cc = oracle_scan(q, k, v1 - 2.5 * v2, u, S0=S1 - 2.5 * S2, **kw)
    np.testing.assert_allclose(cc["o"], a["o"] - 2.5 * b["o"], rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(cc["S"], a["S"] - 2.5 * b["S"], rtol=1e-9, atol=1e-10)
    np.testing.assert_array_equal(a["A"], b["A"])
    # the inverse side is the same as in the additive scan
    np.testing.assert_array_equal(a["A"], oracle_scan(q, k, v1, u, S0=S1, nudge_period=8, eps=1e-3)["A"])
    # resume with the state carried and t0 = T1, cap on
    kw["s_cap"] = 1.5
    full = oracle_scan(q, k, v1, u, **kw)
    assert (full["cap_fires"] > 0).all()
    assert (full["max_s_norm"] <= 1.5 * (1 + 1e-12)).all()
    x = oracle_scan(q[:, :T1], k[:, :T1], v1[:, :T1], u[:, :T1], **kw)
    y = oracle_scan(q[:, T1:], k[:, T1:], v1[:, T1:], u[:, T1:], A0=x["A"], S0=x["S"], n0=x["n"], t0=T1, **kw)
    np.testing.assert_allclose(np.concatenate([x["o"], y["o"]], axis=1), full["o"], rtol=1e-12, atol=1e-14)
    for key in ("A", "S", "n"):
        np.testing.assert_allclose(y[key], full[key], rtol=1e-12, atol=1e-14)


def test_residual_mpmath_brute_force_tiny():
    # 50 digits, direct inverses of the accumulated penalty, the residual
    # state step written from the summary's recursive update rule.
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    C, T, d, r = 2, 10, 4, 2
    q, k, v, u = _rand_inputs(C, T, d, r, seed=39)
    P, cap, eps = 4, 1.2, 1e-2
    res = oracle_scan(q, k, v, u, nudge_period=P, s_cap=cap, eps=eps, update="residual")
    mp = mpmath.mpf
    for c in range(C):
        M = mpmath.eye(d)
        S = mpmath.zeros(d, d)
        n = mpmath.zeros(d, 1)
        nudges = 0
        for t in range(T):
            for i in range(r):
                uu = mpmath.matrix([mp(x) for x in u[c, t, i]])
                M = M + uu * uu.T
            if (t + 1) % P == 0:
                nudges += 1
                # A + eps I = (M^{-1} + eps I): carry M as the inverse of that
                M = (M ** -1 + mp(eps) * mpmath.eye(d)) ** -1
            A = M ** -1
            kk = mpmath.matrix([mp(x) for x in k[c, t]])
            kh = kk / mpmath.sqrt(sum(x * x for x in kk))
            gate = A * kh
            gate = gate / mpmath.sqrt(sum(x * x for x in gate))
            vv = mpmath.matrix([mp(x) for x in v[c, t]])
            S = S + (vv - S * kh) * gate.T
            fn = mpmath.sqrt(sum(S[i, j] ** 2 for i in range(d) for j in range(d)))
            if fn > cap:
                S = S * (mp(cap) / fn)
            n = n + kk
            qq = mpmath.matrix([mp(x) for x in q[c, t]])
            o = S * qq / ((n.T * qq)[0] + mp("1e-6"))
            np.testing.assert_allclose([float(x) for x in o], res["o"][c, t], rtol=1e-11, atol=1e-13)
        assert nudges == T // P
        np.testing.assert_allclose(np.array(S.tolist(), dtype=float), res["S"][c], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(np.array(A.tolist(), dtype=float), res["A"][c], rtol=1e-11, atol=1e-13)

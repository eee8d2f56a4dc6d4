"""GPU parity of the time-parallel schedule at d = 128 (bf16 storage, additive
update, no cap): chunk-boundary inverses from the fp64 Gram prefix and (N, D)
chain, the inverse recurrence per chunk, and the linear state pass (chunk
sums, prefix, chunked readout), against the fp64 oracle."""
import sys

import numpy as np
import pytest
import torch

from recurrent_inverse_scan_amd import CONFIGS, scan_forward
from tests.parity import TOL, case, check, rel_err, run_oracle, to64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(msg):
    print(f"[gpu-chunked128] {msg}", flush=True)
    sys.stdout.flush()


def _gpu(x, cfg, **kw):
    args = dict(nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
    args.update(kw)
    out = scan_forward(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), x["u"].to(DEV), **args)
    torch.cuda.synchronize()
    return out


def _cfg(name, **over):
    return CONFIGS["wide"].with_(name=f"chunked128-{name}", s_cap=None, **over)


CASES = [
    # (name, overrides, chunk_len): ragged state chunks (T not a multiple of
    # 256) and ragged inverse chunks; every rank; nudges inside and at the
    # ends of chunks; a call shorter than one state chunk.
    ("rank4-nudge256", dict(B=1, H=2, T=1000, r=4, nudge_period=256), 128),
    ("rank4-auto-L", dict(B=1, H=3, T=1300, r=4, nudge_period=512), 0),
    ("rank1-nonudge", dict(B=2, H=1, T=700, r=1, nudge_period=0), 64),
    ("rank2-long-chunks", dict(B=1, H=2, T=2100, r=2, nudge_period=1024), 512),
    ("rank3-short", dict(B=1, H=2, T=200, r=3, nudge_period=64), 64),
]


@pytest.mark.parametrize("name,over,L", CASES, ids=[c[0] for c in CASES])
def test_chunked128_matches_oracle(name, over, L):
    cfg = _cfg(name, **over)
    _say(f"case {name} B={cfg.B} H={cfg.H} T={cfg.T} r={cfg.r} P={cfg.nudge_period} L={L}")
    x = case(cfg, seed=21)
    out = _gpu(x, cfg, schedule="chunked", chunk_len=L)
    ref = run_oracle(x, cfg)
    _, st = check("gpu-chunked128", cfg, out, ref, say=_say)
    assert (st[:, 1] == 0).all() and (st[:, 3] == -1).all()


SPANS = [
    # (name, overrides, chunk_len): enough chains that the blocked inverse
    # pass takes spans of four chunks per workgroup, a nudge on every chunk's
    # last token (so one inside each span), and chunks ending in a short
    # block (r = 3: blocks of 10 tokens in 32-token chunks; r = 1: blocks of
    # 32 in 48-token chunks).
    ("rank3-spans", dict(B=2, H=64, T=512, r=3, nudge_period=32), 32),
    ("rank1-spans", dict(B=1, H=128, T=768, r=1, nudge_period=48), 48),
]


@pytest.mark.parametrize("name,over,L", SPANS, ids=[c[0] for c in SPANS])
def test_chunked128_spans_match_oracle(name, over, L):
    cfg = _cfg(name, **over)
    C = cfg.B * cfg.H
    sel = [0, 77, C - 1]
    _say(f"case {name} chains={C} T={cfg.T} r={cfg.r} P={cfg.nudge_period} L={L}, oracle on {sel}")
    x = case(cfg, seed=29)
    out = _gpu(x, cfg, schedule="chunked", chunk_len=L)
    ref = run_oracle(x, cfg, chains=sel)
    check("gpu-chunked128", cfg, out, ref, chains=sel, say=_say)
    seq = _gpu(x, cfg, schedule="sequential")
    for nm, p, q_ in zip("oASn", out[:4], seq[:4]):
        axes = (-2, -1) if nm in "AS" else (-1,)
        err = rel_err(p, to64(q_), axes=axes)
        _say(f"{name}: chunked vs sequential {nm} over all chains: {err}")
        assert err <= (1e-2 if nm == "o" else 1e-4), (nm, err)
    assert torch.equal(out[4], seq[4])


def test_chunked128_spans_ragged_with_state_and_offset():
    """Spans of four chunks where the chain ends in a short span and a short
    chunk (T = 1100, 64-token chunks: 18 chunks), from a given initial state
    at t0 = 192, so the nudges (every 128 tokens) fall at odd chunk ends
    inside the spans; the oracle on sampled chains, the sequential schedule
    on all."""
    cfg = _cfg("spans-ragged", B=2, H=64, T=1100, r=2, nudge_period=128)
    C, d = cfg.B * cfg.H, cfg.d
    sel = [1, 64, C - 1]
    _say(f"case spans-ragged chains={C} T={cfg.T} t0=192, oracle on {sel}")
    x = case(cfg, seed=30)
    g = torch.Generator().manual_seed(30)
    X = torch.randn(C, d, d, generator=g) / d ** 0.5
    A0 = (0.3 * torch.eye(d) + X @ X.transpose(-1, -2) / 4).reshape(cfg.B, cfg.H, d, d).contiguous()
    S0 = torch.randn(cfg.B, cfg.H, d, d, generator=g)
    n0 = torch.rand(cfg.B, cfg.H, d, generator=g)
    t0 = 192
    kw = dict(A0=A0.to(DEV), S0=S0.to(DEV), n0=n0.to(DEV), t0=t0)
    out = _gpu(x, cfg, schedule="chunked", chunk_len=64, **kw)
    ref = run_oracle(x, cfg, chains=sel, A0=A0.reshape(C, d, d)[sel], S0=S0.reshape(C, d, d)[sel],
                     n0=n0.reshape(C, d)[sel], t0=t0)
    check("gpu-chunked128", cfg, out, ref, chains=sel, say=_say)
    seq = _gpu(x, cfg, schedule="sequential", **kw)
    for nm, p, q_ in zip("oASn", out[:4], seq[:4]):
        axes = (-2, -1) if nm in "AS" else (-1,)
        err = rel_err(p, to64(q_), axes=axes)
        _say(f"spans-ragged: chunked vs sequential {nm} over all chains: {err}")
        assert err <= (1e-2 if nm == "o" else 1e-4), (nm, err)
    assert torch.equal(out[4], seq[4])


def test_chunked128_initial_state_and_offset():
    cfg = _cfg("state", B=1, H=2, T=900, r=4, nudge_period=256)
    _say("case initial state, t0 = 512")
    x = case(cfg, seed=22)
    g = torch.Generator().manual_seed(22)
    d = cfg.d
    X = torch.randn(2, d, d, generator=g) / d ** 0.5
    A0 = (0.3 * torch.eye(d) + X @ X.transpose(-1, -2) / 4).reshape(1, 2, d, d).contiguous()
    S0 = torch.randn(1, 2, d, d, generator=g)
    n0 = torch.rand(1, 2, d, generator=g)
    t0 = 512   # a multiple of the chunk length; the nudge phase follows t0
    out = _gpu(x, cfg, A0=A0.to(DEV), S0=S0.to(DEV), n0=n0.to(DEV), t0=t0, schedule="chunked", chunk_len=128)
    ref = run_oracle(x, cfg, A0=A0.reshape(2, d, d), S0=S0.reshape(2, d, d), n0=n0.reshape(2, d), t0=t0)
    check("gpu-chunked128", cfg, out, ref, say=_say)


def test_chunked128_in_place_state_carry():
    """Two calls carrying the state in place (outputs alias the initial
    state) match one oracle run over both halves."""
    cfg = _cfg("inplace", B=1, H=2, T=1024, r=4, nudge_period=256)
    _say("case in-place carry over two calls")
    x = case(cfg, seed=23)
    d = cfg.d
    A = torch.eye(d, device=DEV).expand(1, 2, d, d).contiguous()
    S = torch.zeros(1, 2, d, d, device=DEV)
    n = torch.zeros(1, 2, d, device=DEV)
    st = torch.empty(1, 2, 4, dtype=torch.int32, device=DEV)
    outs = []
    for lo in (0, 512):
        sl = slice(lo, lo + 512)
        q, k, v = (x[nm][:, :, sl].contiguous().to(DEV) for nm in ("q", "k", "v"))
        u = x["u"][:, :, sl].contiguous().to(DEV)
        o = torch.empty_like(q)
        scan_forward(q, k, v, u, A, S, n, nudge_period=256, t0=lo, schedule="chunked", chunk_len=128,
                     out=(o, A, S, n, st))
        outs.append(o)
    torch.cuda.synchronize()
    ref = run_oracle(x, cfg)
    o = torch.cat(outs, dim=2)
    errs = {"o": rel_err(o.reshape(2, cfg.T, d), ref["o"]),
            "A": rel_err(A.reshape(2, d, d), ref["A"], axes=(-2, -1)),
            "S": rel_err(S.reshape(2, d, d), ref["S"], axes=(-2, -1)),
            "n": rel_err(n.reshape(2, d), ref["n"])}
    _say(f"in-place carry: {errs}")
    assert all(v_ <= TOL[cfg.in_dtype] for v_ in errs.values()), errs


def test_chunked128_falls_back_when_the_guard_fires():
    """A Householder start gives delta = 0 on the first token of chain 0: its
    chunk-start inverses are invalid, the chain is flagged and recomputed
    sequentially in the same call, and the guard count matches the oracle."""
    cfg = _cfg("guard", B=1, H=2, T=512, r=1, nudge_period=0)
    _say("case guard fallback")
    x = case(cfg, seed=24)
    d = cfg.d
    u = x["u"].clone()
    e = torch.zeros(d)
    e[5] = 1.0
    u[:, :, 0, 0, :] = e
    x["u"] = u
    A0 = torch.stack([torch.eye(d) - 2 * torch.outer(e, e), torch.eye(d)]).reshape(1, 2, d, d)
    out = _gpu(x, cfg, A0=A0.contiguous().to(DEV), schedule="chunked", chunk_len=128)
    ref = run_oracle(x, cfg, A0=A0.reshape(2, d, d))
    assert list(ref["guard_fires"]) == [1, 0]
    check("gpu-chunked128", cfg, out, ref, say=_say)


def test_chunked128_agrees_with_sequential():
    """The time-parallel and sequential schedules on the wide shape's chain
    length (8192 tokens, rank 4, nudge every 512) agree to fp32 rounding on
    the state and to bf16 rounding on the outputs."""
    cfg = _cfg("vs-seq", B=1, H=4, T=8192, r=4, nudge_period=512)
    _say("case chunked vs sequential, 4 chains of 8192")
    x = case(cfg, seed=25)
    a = _gpu(x, cfg, schedule="chunked")
    b = _gpu(x, cfg, schedule="sequential")
    for name, p, q_ in zip("oASn", a[:4], b[:4]):
        axes = (-2, -1) if name in "AS" else (-1,)
        err = rel_err(p, to64(q_), axes=axes)
        _say(f"chunked vs sequential {name}: {err}")
        assert err <= (1e-2 if name == "o" else 1e-4), (name, err)
    assert torch.equal(a[4], b[4])


def test_chunked128_nonfinite_input_is_flagged():
    """A NaN in v reaches the state pass only: the chain's non-finite flag is
    set, the other chain's is not."""
    cfg = _cfg("nan", B=1, H=2, T=600, r=2, nudge_period=0)
    x = case(cfg, seed=26)
    v = x["v"].clone()
    v[0, 1, 300, 7] = float("nan")
    x["v"] = v
    out = _gpu(x, cfg, schedule="chunked", chunk_len=64)
    st = out[4].reshape(2, 4).cpu().numpy()
    assert st[1, 2] == 1 and st[0, 2] == 0, st
    assert np.isfinite(to64(out[0].reshape(2, cfg.T, cfg.d)[0])).all()


@pytest.mark.parametrize("T", [1, 17, 300])
def test_chunked128_short_calls(T):
    """Calls shorter than one chunk or one 32-token stage (16-token chunks):
    a single token, a ragged 17, and 300 tokens over 19 chunks."""
    cfg = _cfg(f"short-T{T}", B=1, H=2, T=T, r=4, nudge_period=0)
    _say(f"case short call T={T}")
    x = case(cfg, seed=27 + T)
    out = _gpu(x, cfg, schedule="chunked", chunk_len=16)
    check("gpu-chunked128", cfg, out, run_oracle(x, cfg), say=_say)


def test_chunked128_strided_views():
    """q, k, v sliced from one [B, T, H, 3d] tensor (gathered by the library
    into its workspace) give the contiguous call's result bit for bit."""
    cfg = _cfg("strided", B=1, H=3, T=640, r=2, nudge_period=128)
    _say("case strided views")
    x = case(cfg, seed=28)
    d = cfg.d
    packed = torch.cat([x["q"], x["k"], x["v"]], dim=-1).permute(0, 2, 1, 3).contiguous().to(DEV)
    qs, ks, vs = (packed[..., i * d:(i + 1) * d].permute(0, 2, 1, 3) for i in range(3))
    assert not qs.is_contiguous()
    got = scan_forward(qs, ks, vs, x["u"].to(DEV), nudge_period=128, schedule="chunked", chunk_len=128)
    want = _gpu(x, cfg, schedule="chunked", chunk_len=128)
    for a_, b_ in zip(got, want):
        assert torch.equal(a_, b_)
    check("gpu-chunked128", cfg, got, run_oracle(x, cfg), say=_say)

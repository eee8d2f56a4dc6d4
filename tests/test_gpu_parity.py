"""GPU parity: the HIP scan and projection against the fp64 CPU oracle.

Every case calls libvla.so through the C ABI (recurrent_inverse_scan_amd.api)
and compares element by element with the oracle on the same seeded inputs.
The bar is the normwise relative error (per output row, per state matrix):
2e-3 for float32 storage, 1e-2 for bfloat16 storage.
"""
import sys

import numpy as np
import pytest
import torch

from recurrent_inverse_scan_amd import CONFIGS, project_u, scan_forward
from recurrent_inverse_scan_amd._lib import VLAError, VLA_ENONFINITE
from tests.parity import TOL, case, check, flat, oracle_u, rel_err, run_oracle, to64
from oracle.vla_oracle import oracle_project_u, oracle_scan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def _gpu(x, cfg, **kw):
    args = dict(nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
    args.update(kw)
    o, A, S, n, st = scan_forward(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), x["u"].to(DEV), **args)
    torch.cuda.synchronize()
    return o, A, S, n, st


def _check(cfg, out, ref, chains=None, tol=None):
    return check("gpu-parity", cfg, out, ref, chains=chains, tol=tol, say=_say)


# Reduced sizes that the oracle finishes in seconds but that still span several
# LDS stages and a ragged tail (T not a multiple of the stage length).
SMALL = {
    "tiny": CONFIGS["tiny"],
    "base": CONFIGS["base"].with_(B=2, H=3, T=1029),
    "recall": CONFIGS["recall"].with_(B=4, H=8),
    "long": CONFIGS["long"].with_(B=1, H=3, T=2053, nudge_period=64, s_cap=40.0),
    "wide": CONFIGS["wide"].with_(B=1, H=3, T=517, nudge_period=32),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_scan_parity_small(name):
    cfg = SMALL[name]
    _say(f"case small/{name}")
    x = case(cfg)
    out = _gpu(x, cfg)
    ref = run_oracle(x, cfg)
    _, st = _check(cfg, out, ref)
    if cfg.s_cap:
        # cap decisions may differ only where |S|_F is within rounding of the cap
        assert np.abs(st[:, 1] - ref["cap_fires"]).max() <= max(2, 0.01 * ref["cap_fires"].max())


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("r", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_parity_shapes(d, r, dtype):
    cfg = CONFIGS["base"].with_(name=f"shape-d{d}-r{r}", B=1, H=2, T=37, d=d, r=r, in_dtype=dtype,
                                nudge_period=5, s_cap=6.0)
    x = case(cfg, seed=d * 10 + r)
    out = _gpu(x, cfg)
    _check(cfg, out, run_oracle(x, cfg))


# Up to 16 tokens the one-wave kernel runs; beyond, the two-wave kernel with
# 16-token stages at r = 1 (its pipeline fill and drain at 17, 24, 25, 32, 33
# and 40).
@pytest.mark.parametrize("T", [0, 1, 7, 8, 9, 17, 24, 25, 32, 33, 40])
def test_scan_edge_lengths(T):
    cfg = CONFIGS["base"].with_(name=f"len{T}", B=1, H=2, T=T, nudge_period=3, s_cap=5.0)
    x = case(cfg, seed=T)
    g = torch.Generator().manual_seed(T)
    A0 = torch.eye(cfg.d).expand(1, 2, cfg.d, cfg.d) * 0.5 + 0.01 * torch.randn(1, 2, cfg.d, cfg.d, generator=g)
    A0 = ((A0 + A0.transpose(-1, -2)) / 2).contiguous()
    S0 = torch.randn(1, 2, cfg.d, cfg.d, generator=g)
    n0 = torch.rand(1, 2, cfg.d, generator=g)
    out = _gpu(x, cfg, A0=A0.to(DEV), S0=S0.to(DEV), n0=n0.to(DEV), t0=5)
    ref = run_oracle(x, cfg, A0=A0.reshape(2, cfg.d, cfg.d), S0=S0.reshape(2, cfg.d, cfg.d),
                     n0=n0.reshape(2, cfg.d), t0=5)
    _check(cfg, out, ref)
    if T == 0:
        assert torch.equal(out[1].cpu(), A0) and torch.equal(out[2].cpu(), S0) and torch.equal(out[3].cpu(), n0)


def test_guard_fire_householder_start():
    """A0 = I - 2 u u^T with u the first direction: delta = 0 exactly, the guard fires."""
    cfg = CONFIGS["base"].with_(name="guard", B=1, H=2, T=20, nudge_period=0, s_cap=None)
    x = case(cfg, seed=3)
    u = x["u"].clone()
    e = torch.zeros(cfg.d)
    e[5] = 1.0
    u[:, :, 0, 0, :] = e
    x["u"] = u
    A0 = (torch.eye(cfg.d) - 2 * torch.outer(e, e)).expand(1, 2, cfg.d, cfg.d).contiguous()
    out = _gpu(x, cfg, A0=A0.to(DEV))
    ref = run_oracle(x, cfg, A0=A0.reshape(2, cfg.d, cfg.d))
    assert (ref["guard_fires"] == 1).all()
    _check(cfg, out, ref)


# For r > 1 the kernels apply a token's r rank-1 updates as one rank-r update
# unless a delta trips the guard; then the token runs them one at a time.
@pytest.mark.parametrize("d,T", [(64, 20), (64, 5), (128, 20)])
@pytest.mark.parametrize("r,at", [(2, 0), (2, 1), (3, 1), (4, 2)])
def test_guard_fire_in_a_rank_r_token(d, T, r, at):
    """A0 = I - 2 e e^T; direction `at` of the first token is e and the earlier
    ones are orthogonal unit vectors, so that direction's delta is exactly 0."""
    cfg = CONFIGS["base"].with_(name=f"guard-r{r}-at{at}-d{d}-T{T}", B=1, H=2, T=T, d=d, r=r, nudge_period=0,
                                s_cap=None)
    x = case(cfg, seed=40 + r + at)
    u = x["u"].clone()
    eye = torch.eye(d)
    for j in range(at):
        u[:, :, 0, j, :] = eye[11 + j]
    u[:, :, 0, at, :] = eye[5]
    x["u"] = u
    A0 = (eye - 2 * torch.outer(eye[5], eye[5])).expand(1, 2, d, d).contiguous()
    out = _gpu(x, cfg, A0=A0.to(DEV))
    ref = run_oracle(x, cfg, A0=A0.reshape(2, d, d))
    assert (ref["guard_fires"] == 1).all()
    _check(cfg, out, ref)


def test_cap_forced_every_step():
    cfg = CONFIGS["base"].with_(name="cap1", B=1, H=2, T=50, nudge_period=0, s_cap=1.0)
    x = case(cfg, seed=4)
    out = _gpu(x, cfg)
    ref = run_oracle(x, cfg)
    _, st = _check(cfg, out, ref)
    assert (st[:, 1] == cfg.T).all() and (st[:, 3] == 0).all()
    assert (np.linalg.norm(to64(out[2]), axis=(-2, -1)) <= 1.0 + 1e-5).all()


def test_resume_and_in_place_state_carry():
    cfg = CONFIGS["base"].with_(name="resume", B=1, H=2, T=200)
    x = case(cfg, seed=5)
    full = _gpu(x, cfg)
    T1 = 77
    q, k, v, u = (x[n].to(DEV) for n in ("q", "k", "v", "u"))
    o1, A, S, n, _ = scan_forward(q[:, :, :T1].contiguous(), k[:, :, :T1].contiguous(), v[:, :, :T1].contiguous(),
                                  u[:, :, :T1].contiguous(), nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
    st = torch.empty((1, 2, 4), dtype=torch.int32, device=DEV)
    o2 = torch.empty_like(q[:, :, T1:])
    scan_forward(q[:, :, T1:].contiguous(), k[:, :, T1:].contiguous(), v[:, :, T1:].contiguous(),
                 u[:, :, T1:].contiguous(), A, S, n, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, t0=T1,
                 out=(o2, A, S, n, st))
    torch.cuda.synchronize()
    ref = run_oracle(x, cfg)
    assert rel_err(torch.cat([o1, o2], dim=2).reshape(2, cfg.T, cfg.d), ref["o"]) <= 2e-3
    assert rel_err(A.reshape(2, cfg.d, cfg.d), ref["A"], axes=(-2, -1)) <= 2e-3
    assert rel_err(S.reshape(2, cfg.d, cfg.d), ref["S"], axes=(-2, -1)) <= 2e-3
    # split and unsplit runs agree closely (same arithmetic, state round-tripped through HBM)
    assert rel_err(torch.cat([o1, o2], dim=2), to64(full[0])) <= 1e-5


def test_nonfinite_flag_and_validate():
    cfg = CONFIGS["base"].with_(name="nan", B=1, H=2, T=40)
    x = case(cfg, seed=6)
    v = x["v"].clone()
    v[0, 1, 10, 3] = float("nan")
    x["v"] = v
    out = _gpu(x, cfg)
    st = out[4].cpu().numpy().reshape(2, 4)
    assert list(st[:, 2]) == [0, 1]
    with pytest.raises(VLAError) as ei:
        scan_forward(x["q"].to(DEV), x["k"].to(DEV), v.to(DEV), x["u"].to(DEV), validate=True)
    assert ei.value.status == VLA_ENONFINITE
    clean = case(cfg, seed=6)
    scan_forward(clean["q"].to(DEV), clean["k"].to(DEV), clean["v"].to(DEV), clean["u"].to(DEV), validate=True)


def test_bitwise_repeatable():
    cfg = CONFIGS["base"].with_(name="repeat", B=2, H=2, T=300)
    x = case(cfg, seed=7)
    a = _gpu(x, cfg)
    b = _gpu(x, cfg)
    for p, q_ in zip(a, b):
        assert torch.equal(p, q_)


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("r", [1, 3, 4])
@pytest.mark.parametrize("din,dout", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16")])
def test_project_u_parity(d, r, din, dout):
    g = torch.Generator().manual_seed(d + r)
    # Several 128-row workgroups, several runs of 8 or 16 row tiles per wave
    # (bf16 kernel) with a short last run, and a ragged tail.
    rows = 1000 + 37
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    W = (torch.randn(r, d, d, generator=g) / d ** 0.5).to(dt[din])
    kr = torch.randn(rows, d, generator=g).to(dt[din])
    kr[3] = 0.0        # a zero row stays zero
    u = project_u(W.to(DEV), kr.to(DEV), out_dtype=dt[dout])
    torch.cuda.synchronize()
    ref = oracle_project_u(W, kr)
    tol = 2e-3 if dout == "f32" else 1e-2
    err = rel_err(u.reshape(rows * r, d), ref.reshape(rows * r, d))
    _say(f"project d={d} r={r} {din}->{dout}: {err}")
    assert err <= (1e-5 if (din, dout) == ("f32", "f32") else tol)
    assert (u[3] == 0).all()


# ---------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times (GPU
# projection then scan on all chains); the oracle runs on sampled chains.
# ---------------------------------------------------------------------------
FULL_SAMPLES = {"tiny": None, "base": [0, 31], "recall": [0, 511], "long": [0, 15], "wide": [0, 127]}


@pytest.mark.parametrize("name", list(FULL_SAMPLES))
def test_full_size_sampled_chains(name):
    cfg = CONFIGS[name]
    chains = FULL_SAMPLES[name]
    _say(f"case full/{name} chains={chains}")
    from recurrent_inverse_scan_amd import make_inputs

    x = make_inputs(cfg, seed=0)
    u = project_u(x["W_u"].to(DEV), x["k_raw"].to(DEV))
    o, A, S, n, st = scan_forward(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), u,
                                  nudge_period=cfg.nudge_period, s_cap=cfg.s_cap)
    torch.cuda.synchronize()
    C = cfg.B * cfg.H
    sel = list(range(C)) if chains is None else chains
    kr = x["k_raw"].reshape(C, cfg.T, cfg.d)[sel]
    u_ref = oracle_project_u(x["W_u"], kr.reshape(-1, cfg.d))
    u_ref = torch.from_numpy(u_ref).to(x["q"].dtype).reshape(len(sel), cfg.T, cfg.r, cfg.d)
    ref = oracle_scan(x["q"].reshape(C, cfg.T, cfg.d)[sel], x["k"].reshape(C, cfg.T, cfg.d)[sel],
                      x["v"].reshape(C, cfg.T, cfg.d)[sel], u_ref, nudge_period=cfg.nudge_period,
                      s_cap=cfg.s_cap, trace_norms=True)
    _, st = _check(cfg, (o, A, S, n, st), ref, chains=sel)
    if cfg.s_cap:
        # cap decisions may differ only where |S|_F is within rounding of the cap
        _say(f"cap fires gpu {st[:, 1].tolist()} oracle {ref['cap_fires'].tolist()}")
        assert np.abs(st[:, 1] - ref["cap_fires"]).max() <= max(2, 0.01 * ref["cap_fires"].max())


def test_full_size_long_repeatable_on_reused_buffers():
    """The long workload, run twice on the same workspace and output buffers
    exactly as the benchmark does, gives bit-identical results."""
    from recurrent_inverse_scan_amd import make_inputs, workspace_size

    cfg = CONFIGS["long"]
    _say("case full/long repeat")
    x = make_inputs(cfg, seed=0)
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    u = project_u(x["W_u"].to(DEV), x["k_raw"].to(DEV))
    B, H, d = cfg.B, cfg.H, cfg.d
    outs = (torch.empty_like(q), torch.empty((B, H, d, d), device=DEV), torch.empty((B, H, d, d), device=DEV),
            torch.empty((B, H, d), device=DEV), torch.empty((B, H, 4), device=DEV, dtype=torch.int32))
    ws = torch.empty(workspace_size(B, H, cfg.T, d, cfg.r, q.dtype, nudge_period=cfg.nudge_period,
                                    s_cap=cfg.s_cap), device=DEV, dtype=torch.uint8)
    runs = []
    for _ in range(3):
        scan_forward(q, k, v, u, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, out=outs, workspace=ws)
        torch.cuda.synchronize()
        runs.append([t.clone() for t in outs])
    for later in runs[1:]:
        for a, b in zip(runs[0], later):
            assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# Time-parallel (chunked) schedule.
# ---------------------------------------------------------------------------
CHUNKED = [
    # (name, overrides, chunk_len)
    ("f32-nudge", dict(B=1, H=3, T=1000, in_dtype="f32", nudge_period=128, s_cap=None), 64),
    ("bf16-nudge-cap", dict(B=2, H=2, T=777, in_dtype="bf16", nudge_period=64, s_cap=25.0), 64),
    ("f32-rank3", dict(B=1, H=2, T=300, r=3, in_dtype="f32", nudge_period=32, s_cap=None), 32),
    ("bf16-rank4-nonudge", dict(B=1, H=2, T=333, r=4, in_dtype="bf16", nudge_period=0, s_cap=None), 64),
    ("f32-cap-binding", dict(B=1, H=2, T=513, in_dtype="f32", nudge_period=0, s_cap=3.0), 128),
    # One direction per token takes the blocked (32-token) inverse pass: a
    # chunk of 48 ends in a half block, and the last chunk is ragged.
    ("bf16-blocked-half-block", dict(B=1, H=2, T=500, in_dtype="bf16", nudge_period=96, s_cap=30.0), 48),
    ("f32-blocked-half-block", dict(B=1, H=2, T=500, in_dtype="f32", nudge_period=96, s_cap=30.0), 48),
    # Long chunks with the nudge on every other chunk's last token.
    ("bf16-blocked-long-chunks", dict(B=1, H=2, T=2100, in_dtype="bf16", nudge_period=1024, s_cap=None), 512),
    ("f32-blocked-long-chunks", dict(B=1, H=2, T=2100, in_dtype="f32", nudge_period=1024, s_cap=None), 512),
]


@pytest.mark.parametrize("name,over,L", CHUNKED, ids=[c[0] for c in CHUNKED])
def test_chunked_matches_oracle(name, over, L):
    cfg = CONFIGS["base"].with_(name=f"chunked-{name}", **over)
    _say(f"case chunked/{name}")
    x = case(cfg, seed=11)
    out = _gpu(x, cfg, schedule="chunked", chunk_len=L)
    ref = run_oracle(x, cfg)
    _, st = _check(cfg, out, ref)
    if cfg.s_cap:
        assert np.abs(st[:, 1] - ref["cap_fires"]).max() <= max(2, 0.01 * ref["cap_fires"].max())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunked_with_initial_state_and_offset(dtype):
    cfg = CONFIGS["base"].with_(name=f"chunked-state-{dtype}", B=1, H=2, T=640, in_dtype=dtype, nudge_period=128,
                                s_cap=50.0)
    x = case(cfg, seed=12)
    g = torch.Generator().manual_seed(12)
    X = torch.randn(2, cfg.d, cfg.d, generator=g) / cfg.d ** 0.5
    A0 = (0.3 * torch.eye(cfg.d) + X @ X.transpose(-1, -2) / 4).reshape(1, 2, cfg.d, cfg.d).contiguous()
    S0 = torch.randn(1, 2, cfg.d, cfg.d, generator=g)
    n0 = torch.rand(1, 2, cfg.d, generator=g)
    t0 = 256   # a multiple of the chunk length; the nudge phase follows t0
    out = _gpu(x, cfg, A0=A0.to(DEV), S0=S0.to(DEV), n0=n0.to(DEV), t0=t0, schedule="chunked", chunk_len=64)
    ref = run_oracle(x, cfg, A0=A0.reshape(2, cfg.d, cfg.d), S0=S0.reshape(2, cfg.d, cfg.d),
                     n0=n0.reshape(2, cfg.d), t0=t0)
    _check(cfg, out, ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunked_in_place_state_carry(dtype):
    cfg = CONFIGS["base"].with_(name=f"chunked-inplace-{dtype}", B=1, H=2, T=512, in_dtype=dtype, nudge_period=64,
                                s_cap=None)
    x = case(cfg, seed=13)
    q, k, v, u = (x[n].to(DEV) for n in ("q", "k", "v", "u"))
    A = torch.eye(cfg.d, device=DEV).expand(1, 2, cfg.d, cfg.d).contiguous()
    S = torch.zeros(1, 2, cfg.d, cfg.d, device=DEV)
    n = torch.zeros(1, 2, cfg.d, device=DEV)
    st = torch.empty(1, 2, 4, dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    scan_forward(q, k, v, u, A, S, n, nudge_period=64, schedule="chunked", chunk_len=64, out=(o, A, S, n, st))
    torch.cuda.synchronize()
    ref = run_oracle(x, cfg)
    assert rel_err(o.reshape(2, cfg.T, cfg.d), ref["o"]) <= TOL[cfg.in_dtype]
    assert rel_err(A.reshape(2, cfg.d, cfg.d), ref["A"], axes=(-2, -1)) <= 2e-3
    assert rel_err(S.reshape(2, cfg.d, cfg.d), ref["S"], axes=(-2, -1)) <= 2e-3


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunked_falls_back_when_the_guard_fires(dtype):
    """A Householder start makes delta = 0 in the first chunk: the chain is
    recomputed sequentially inside the same call and still matches."""
    cfg = CONFIGS["base"].with_(name=f"chunked-guard-{dtype}", B=1, H=2, T=256, in_dtype=dtype, nudge_period=0,
                                s_cap=None)
    x = case(cfg, seed=14)
    u = x["u"].clone()
    e = torch.zeros(cfg.d)
    e[7] = 1.0
    u[:, :, 0, 0, :] = e
    x["u"] = u
    A0 = torch.stack([torch.eye(cfg.d) - 2 * torch.outer(e, e), torch.eye(cfg.d)]).reshape(1, 2, cfg.d, cfg.d)
    out = _gpu(x, cfg, A0=A0.contiguous().to(DEV), schedule="chunked", chunk_len=64)
    ref = run_oracle(x, cfg, A0=A0.reshape(2, cfg.d, cfg.d))
    assert list(ref["guard_fires"]) == [1, 0]
    _check(cfg, out, ref)


def test_chunked_agrees_with_sequential():
    cfg = CONFIGS["long"].with_(name="chunked-vs-seq", B=1, H=4, T=4096)
    x = case(cfg, seed=15)
    a = _gpu(x, cfg, schedule="chunked", chunk_len=512)
    b = _gpu(x, cfg, schedule="sequential")
    for name, p, q_ in zip("oASn", a[:4], b[:4]):
        axes = (-2, -1) if name in "AS" else (-1,)
        err = rel_err(p, to64(q_), axes=axes)
        _say(f"chunked vs sequential {name}: {err}")
        assert err <= (1e-2 if name == "o" else 1e-3), (name, err)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L,period,seg", [(64, 128, 2), (64, 128, 6), (64, 128, 10), (128, 128, 3), (96, 192, 5)])
def test_chunked_segments_match_oracle(dtype, L, period, seg):
    """The per-chain pass cut into segments (seg rounds up to 4, 8, 12, 4 and
    8 blocks here; over the 32 blocks of T = 2000 that gives segments of
    2 4 4 4 4 4 4 4 2, 6 8 8 6 4 and 8 12 12 blocks: a short first segment,
    a remainder shared with the segment before, and boundaries inside chunks
    for L = 96 and 128), the next segment's prep and the last one's readout on
    the side stream: every segment boundary carries S, n and the cap counters;
    outputs match the oracle."""
    cfg = CONFIGS["base"].with_(name=f"chunked-L{L}-seg{seg}-{dtype}", B=1, H=3, T=2000, in_dtype=dtype,
                                nudge_period=period, s_cap=30.0)
    _say(f"case chunked L={L} segments {seg} {dtype}")
    x = case(cfg, seed=16)
    out = _gpu(x, cfg, schedule="chunked", chunk_len=L, segment_blocks=seg, para_segments=1)
    ref = run_oracle(x, cfg)
    _, st = _check(cfg, out, ref)
    assert ref["cap_fires"].min() > 10
    assert np.abs(st[:, 1] - ref["cap_fires"]).max() <= max(2, 0.01 * ref["cap_fires"].max())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,seg", [(438, 2), (30000, 0)])
def test_chunked_segment_with_odd_start_block(dtype, T, seg):
    """A remainder shared between the last two segments can start the last
    one at an odd block: T = 438 (7 blocks of 64) with seg = 2 gives
    segments [0, 2, 5, 7], and T = 30000 (469 blocks) with the default
    length gives [0, 160, 341, 469].  The cap fires all through the last two
    blocks, so the final state depends on the last block's weights and
    scale, which the last segment must take from the buffer of its parity
    relative to its own first block."""
    cfg = CONFIGS["base"].with_(name=f"chunked-odd-{T}-{dtype}", B=1, H=2, T=T, in_dtype=dtype, nudge_period=128,
                                s_cap=3.0)
    _say(f"case chunked odd segment start T={T} seg={seg} {dtype}")
    x = case(cfg, seed=17)
    out = _gpu(x, cfg, schedule="chunked", chunk_len=64, segment_blocks=seg, para_segments=1)
    ref = run_oracle(x, cfg)
    _, st = _check(cfg, out, ref)
    assert ref["cap_fires"].min() > T // 2
    assert np.abs(st[:, 1] - ref["cap_fires"]).max() <= max(2, 0.01 * ref["cap_fires"].max())


def test_timing_hook_records_the_chain_kernel():
    """The measurement hook returns positive durations, the same number of
    chain-kernel launches for every chunked scan."""
    from recurrent_inverse_scan_amd import timing_collect, timing_enable

    cfg = CONFIGS["base"].with_(name="timing", B=1, H=2, T=640, nudge_period=128, s_cap=50.0)
    x = case(cfg, seed=3)
    timing_enable(True)
    try:
        for _ in range(3):
            _gpu(x, cfg, schedule="chunked")
        ms = timing_collect()
    finally:
        timing_enable(False)
    _say(f"chain kernel ms {ms}")
    assert len(ms) >= 3 and len(ms) % 3 == 0 and all(t > 0 for t in ms)
    assert timing_collect() == []
    timing_enable(True)
    try:
        for _ in range(2):
            # one pass per chain, 10 blocks: segments of 2, 4, 4
            _gpu(x, cfg, schedule="chunked", segment_blocks=4, para_segments=1)
        ms = timing_collect()
    finally:
        timing_enable(False)
    assert len(ms) == 6 and all(t > 0 for t in ms), ms
    timing_enable(True)
    try:
        # parallel in time, 5 segments: at most 5 passes (then the segment
        # starts are exact)
        _gpu(x, cfg, schedule="chunked", para_segments=5)
        ms = timing_collect()
    finally:
        timing_enable(False)
    assert len(ms) == 5 and all(t > 0 for t in ms), ms


# Short calls (T <= 16 tokens, the decode-like case) run the full scan with
# more waves per chain at d = 32 and 64; both updates, from a carried state.
@pytest.mark.parametrize("update", ["additive", "residual"])
@pytest.mark.parametrize("d,r,dtype", [(16, 1, "f32"), (32, 3, "bf16"), (64, 1, "bf16"), (64, 4, "f32"),
                                       (128, 2, "bf16")])
@pytest.mark.parametrize("T", [1, 5, 16])
def test_short_calls_match_oracle(update, d, r, dtype, T):
    cfg = CONFIGS["base"].with_(name=f"short-{update}-d{d}-r{r}-{dtype}-T{T}", B=3, H=5, T=T, d=d, r=r,
                                in_dtype=dtype, nudge_period=4, s_cap=25.0)
    x = case(cfg, seed=T * 100 + d + r)
    g = torch.Generator().manual_seed(d + T)
    C = cfg.B * cfg.H
    A0 = torch.eye(d).expand(cfg.B, cfg.H, d, d) * 0.7 + 0.02 * torch.randn(cfg.B, cfg.H, d, d, generator=g)
    A0 = ((A0 + A0.transpose(-1, -2)) / 2).contiguous()
    S0 = torch.randn(cfg.B, cfg.H, d, d, generator=g)
    n0 = torch.rand(cfg.B, cfg.H, d, generator=g) * 10
    out = _gpu(x, cfg, A0=A0.to(DEV), S0=S0.to(DEV), n0=n0.to(DEV), t0=3, update=update)
    ref = run_oracle(x, cfg, A0=A0.reshape(C, d, d), S0=S0.reshape(C, d, d), n0=n0.reshape(C, d), t0=3,
                     update=update)
    _check(cfg, out, ref)


# One-token calls at d = 64 run a dedicated decode kernel.
@pytest.mark.parametrize("update", ["additive", "residual"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_guard_fire_householder_start(update, dtype):
    """T = 1 from A0 = I - 2 u u^T with u the token's direction: delta = 0
    exactly, so the guard fires in the decode kernel too."""
    cfg = CONFIGS["base"].with_(name=f"decode-guard-{update}-{dtype}", B=2, H=3, T=1, nudge_period=0, s_cap=None,
                                in_dtype=dtype)
    x = case(cfg, seed=31)
    e = torch.zeros(cfg.d)
    e[9] = 1.0
    u = x["u"].clone()
    u[:, :, 0, 0, :] = e.to(u.dtype)
    x["u"] = u
    A0 = (torch.eye(cfg.d) - 2 * torch.outer(e, e)).expand(cfg.B, cfg.H, cfg.d, cfg.d).contiguous()
    out = _gpu(x, cfg, A0=A0.to(DEV), update=update)
    ref = run_oracle(x, cfg, A0=A0.reshape(cfg.B * cfg.H, cfg.d, cfg.d), update=update)
    assert (ref["guard_fires"] == 1).all()
    _check(cfg, out, ref)


@pytest.mark.parametrize("update", ["additive", "residual"])
def test_decode_steps_match_one_call(update):
    """Twenty-four one-token calls with the state carried in place (A_T, S_T,
    n_T aliasing A0, S0, n0; t0 advancing, so the nudge phase moves) equal one
    24-token call and the oracle."""
    cfg = CONFIGS["long"].with_(name=f"decode-steps-{update}", B=4, H=8, T=24, nudge_period=5, s_cap=12.0)
    x = case(cfg, seed=32)
    whole = _gpu(x, cfg, update=update)
    B, H, d = cfg.B, cfg.H, cfg.d
    A = torch.eye(d, device=DEV).expand(B, H, d, d).contiguous()
    S = torch.zeros(B, H, d, d, device=DEV)
    n = torch.zeros(B, H, d, device=DEV)
    st = torch.empty(B, H, 4, device=DEV, dtype=torch.int32)
    outs, fires = [], 0
    for t in range(cfg.T):
        sl = {key: x[key][:, :, t:t + 1].contiguous().to(DEV) for key in ("q", "k", "v", "u")}
        o = torch.empty_like(sl["q"])
        scan_forward(sl["q"], sl["k"], sl["v"], sl["u"], A, S, n, nudge_period=cfg.nudge_period, s_cap=cfg.s_cap,
                     t0=t, update=update, out=(o, A, S, n, st))
        torch.cuda.synchronize()
        fires += st[..., 1].cpu().numpy()
        outs.append(o)
    o_steps = torch.cat(outs, dim=2)
    ref = run_oracle(x, cfg, update=update)
    _check(cfg, (o_steps, A, S, n, whole[4]), ref)
    assert rel_err(o_steps, whole[0].float().cpu().numpy()) <= 1e-2
    assert np.abs(fires.reshape(-1) - ref["cap_fires"]).max() <= 1


# ---------------------------------------------------------------------------
# Strided q, k, v (views of one packed projection) and the decode entry point.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("schedule,T", [("sequential", 77), ("chunked", 640), ("auto", 1)])
def test_strided_views_of_a_packed_projection(dtype, schedule, T):
    """q, k, v sliced from one [B, T, H, 3d] tensor and permuted to
    [B, H, T, d] views (strides T*H*3d, 3d, H*3d) give the same result as
    contiguous copies, and match the oracle."""
    cfg = CONFIGS["base"].with_(name=f"strided-{schedule}-{dtype}-T{T}", B=2, H=3, T=T, in_dtype=dtype,
                                nudge_period=64 if T > 1 else 0, s_cap=40.0)
    _say(f"case strided {schedule} {dtype} T={T}")
    x = case(cfg, seed=50 + T)
    d = cfg.d
    packed = torch.cat([x["q"], x["k"], x["v"]], dim=-1).permute(0, 2, 1, 3).contiguous().to(DEV)  # [B,T,H,3d]
    qs, ks, vs = (packed[..., i * d:(i + 1) * d].permute(0, 2, 1, 3) for i in range(3))
    assert not qs.is_contiguous() and qs.stride()[:2] == (T * cfg.H * 3 * d, 3 * d) and qs.stride(3) == 1
    assert T == 1 or qs.stride(2) == cfg.H * 3 * d   # (torch normalises a size-1 dimension's stride)
    kw = dict(nudge_period=cfg.nudge_period, s_cap=cfg.s_cap, schedule=schedule)
    if schedule == "chunked":
        kw["chunk_len"] = 64
    got = scan_forward(qs, ks, vs, x["u"].to(DEV), **kw)
    want = _gpu(x, cfg, schedule=schedule, **({"chunk_len": 64} if schedule == "chunked" else {}))
    for a_, b_ in zip(got, want):
        assert torch.equal(a_, b_)
    _check(cfg, got, run_oracle(x, cfg))


@pytest.mark.parametrize("update", ["additive", "residual"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_step_entry_point(update, dtype):
    """vla_scan_step over 20 tokens (state in place, t0 advancing through
    nudges) equals the oracle's 20-token scan and one vla_scan_forward call."""
    from recurrent_inverse_scan_amd import scan_step

    cfg = CONFIGS["long"].with_(name=f"step-{update}-{dtype}", B=3, H=4, T=20, in_dtype=dtype, nudge_period=6,
                                s_cap=10.0)
    x = case(cfg, seed=60)
    B, H, d = cfg.B, cfg.H, cfg.d
    A = torch.eye(d, device=DEV).expand(B, H, d, d).contiguous()
    S = torch.zeros(B, H, d, d, device=DEV)
    n = torch.zeros(B, H, d, device=DEV)
    outs, fires = [], 0
    for t in range(cfg.T):
        sl = {key: x[key][:, :, t:t + 1].contiguous().to(DEV) for key in ("q", "k", "v", "u")}
        o, st = scan_step(sl["q"], sl["k"], sl["v"], sl["u"], A, S, n, nudge_period=cfg.nudge_period,
                          s_cap=cfg.s_cap, t0=t, update=update)
        torch.cuda.synchronize()
        fires = fires + st[..., 1].cpu().numpy()
        outs.append(o)
    whole = _gpu(x, cfg, update=update)
    ref = run_oracle(x, cfg, update=update)
    _check(cfg, (torch.cat(outs, dim=2), A, S, n, whole[4]), ref)
    assert np.abs(fires.reshape(-1) - ref["cap_fires"]).max() <= 1


# ---------------------------------------------------------------------------
# Parallel-in-time state pass: segments of each chain run at once from guessed
# starts and are corrected by sweeps (the default for few chains); the
# one-pass pipeline (para_segments = 1) is the reference schedule.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("G,cap,T", [(2, 30.0, 1000), (5, 30.0, 2000), (16, 30.0, 3000), (16, None, 3000),
                                     (8, 3.0, 1500), (16, 1e3, 9000)])
def test_parallel_in_time_state_pass(dtype, G, cap, T):
    """Against the oracle, and against the one-pass pipeline on the same
    inputs: caps that bind early (30, 3: the sweeps must turn the starts
    through many fires), no cap (the first sweep is already exact), a cap
    that starts binding part-way (1e3 over 9000 tokens)."""
    cfg = CONFIGS["long"].with_(name=f"para-G{G}-cap{cap}-{dtype}-T{T}", B=1, H=3, T=T, in_dtype=dtype,
                                nudge_period=128, s_cap=cap)
    _say(f"case para G={G} cap={cap} T={T} {dtype}")
    x = case(cfg, seed=18 + G)
    out = _gpu(x, cfg, schedule="chunked", chunk_len=64, para_segments=G)
    ref = run_oracle(x, cfg)
    _check(cfg, out, ref)
    one = _gpu(x, cfg, schedule="chunked", chunk_len=64, para_segments=1)
    for name, p_, q_ in zip("oASn", out[:4], one[:4]):
        axes = (-2, -1) if name in "AS" else (-1,)
        err = rel_err(p_, to64(q_), axes=axes)
        assert err <= (1e-2 if name == "o" else 2e-4), (name, err)

"""Seeded synthetic workloads for the VLA scan.

This module only draws random inputs and casts them to their storage dtype.
It holds none of the scan's arithmetic and none of the projection's: the
penalty directions u are computed from ``W_u`` and ``k_raw`` by whichever side
consumes them (the HIP library, or the fp64 oracle in tests).

Recipe (shared by tests, the smoke check and the benchmark):

* one CPU ``torch.Generator`` seeded with ``seed`` (0 by default);
* Gaussian workloads draw, in this order: q_raw, k_raw, v as [B, H, T, d]
  standard normals, then W_u as [r, d, d] normals with variance 1/d;
* q = ELU(q_raw) + 1 and k = ELU(k_raw) + 1 are the positive feature map
  ("Variational Linear Attention (VLA)" README, v3 notes item 1), applied in
  float32 before any cast to the storage dtype;
* the associative-recall workload stands in for the pages' multi-query
  associative recall task (no dataset is used): each (b, h) chain is one
  sequence with its own pool of 24 random unit key vectors and 24 N(0, 1)
  value vectors; at every position a pool index j ~ U{0..23} is drawn,
  k_raw = p_j + N(0, 0.01) noise and v = w_j; queries are ELU(N(0,1)) + 1,
  except the last 128 positions, whose queries are a re-presented pool key
  ELU(p_j' + fresh noise) + 1 with j' ~ U{0..23}.  Draw order: q_raw, pool,
  values, key indices, key noise, query indices, query noise, W_u;
* casts to bfloat16 round to nearest even (torch's default).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

__all__ = ["ScanConfig", "CONFIGS", "make_inputs", "storage_dtype"]


@dataclasses.dataclass(frozen=True)
class ScanConfig:
    name: str
    B: int
    H: int
    T: int
    d: int
    r: int
    in_dtype: str            # "f32" or "bf16": storage of q, k, v, u, k_raw, W_u and o
    nudge_period: int        # 0 = off
    s_cap: Optional[float]   # None = off
    kind: str = "gaussian"   # "gaussian" or "recall"

    @property
    def chains(self) -> int:
        return self.B * self.H

    def with_(self, **kw) -> "ScanConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": ScanConfig("tiny", 1, 1, 256, 16, 1, "f32", 0, None),
    "base": ScanConfig("base", 4, 8, 2048, 64, 1, "f32", 256, 1e3),
    "recall": ScanConfig("recall", 64, 8, 512, 64, 1, "f32", 0, None, kind="recall"),
    "long": ScanConfig("long", 2, 8, 65536, 64, 1, "bf16", 1024, 1e3),
    "wide": ScanConfig("wide", 8, 16, 8192, 128, 4, "bf16", 512, None),
}


def storage_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _feature(x: torch.Tensor) -> torch.Tensor:
    return torch.nn.functional.elu(x) + 1.0


def make_inputs(cfg: ScanConfig, seed: int = 0):
    """Return a dict of CPU tensors in the storage dtype.

    Keys: q, k, v [B, H, T, d]; q_raw, k_raw [B, H, T, d]; W_u [r, d, d].
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    B, H, T, d, r = cfg.B, cfg.H, cfg.T, cfg.d, cfg.r
    shape = (B, H, T, d)
    if cfg.kind == "gaussian":
        q_raw = torch.randn(shape, generator=g, dtype=torch.float32)
        k_raw = torch.randn(shape, generator=g, dtype=torch.float32)
        v = torch.randn(shape, generator=g, dtype=torch.float32)
        q = _feature(q_raw)
    elif cfg.kind == "recall":
        npool = 24
        q_raw = torch.randn(shape, generator=g, dtype=torch.float32)
        pool = torch.randn((B, H, npool, d), generator=g, dtype=torch.float32)
        pool = pool / pool.norm(dim=-1, keepdim=True)
        vals = torch.randn((B, H, npool, d), generator=g, dtype=torch.float32)
        idx = torch.randint(0, npool, (B, H, T), generator=g)
        knoise = 0.1 * torch.randn(shape, generator=g, dtype=torch.float32)
        nq = min(128, T)
        qidx = torch.randint(0, npool, (B, H, nq), generator=g)
        qnoise = 0.1 * torch.randn((B, H, nq, d), generator=g, dtype=torch.float32)
        gather = lambda src, ix: torch.gather(src, 2, ix[..., None].expand(*ix.shape, d))
        k_raw = gather(pool, idx) + knoise
        v = gather(vals, idx)
        q_raw[:, :, T - nq:, :] = gather(pool, qidx) + qnoise
        q = _feature(q_raw)
    else:
        raise ValueError(f"unknown workload kind {cfg.kind!r}")
    W_u = torch.randn((r, d, d), generator=g, dtype=torch.float32) / math.sqrt(d)
    k = _feature(k_raw)
    dt = storage_dtype(cfg.in_dtype)
    return {
        "q": q.to(dt).contiguous(),
        "k": k.to(dt).contiguous(),
        "v": v.to(dt).contiguous(),
        "q_raw": q_raw.to(dt).contiguous(),
        "k_raw": k_raw.to(dt).contiguous(),
        "W_u": W_u.to(dt).contiguous(),
    }

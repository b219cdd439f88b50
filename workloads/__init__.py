"""Seeded synthetic decode-step inputs for SANTA / S²ANTA attention.

This module only builds inputs: it holds none of the method's arithmetic, and both the HIP path's
tests and the CPU oracle read the arrays it returns. Generation runs on the host with numpy's PCG64,
so the same seed gives the same inputs on every machine; values are drawn in fp32 and then cast to
the compute dtype (bf16, round-to-nearest-even) with torch.

The kernel benchmark in "Stochastic Sparse Attention for Memory-Bound Inference" (Appendix Q) uses
i.i.d. Gaussian q, K, V at Llama-3.1-8B shapes (H=32, Hkv=8, dk=128) with a sequence-major
[nk, Hkv, dk] cache. The workloads here add planted keys aligned with the queries so the softmax is
peaked, standing in for the real long-context attention the pages' accuracy studies use (those
prompts and models are not used here):

  * planted spikes: per (batch, query head h), P positions (distinct across the G heads of a KV group)
    get K = r * (0.9 * q_h/|q_h| + sqrt(0.19) * w), with w a random unit vector orthogonal to q_h and
    r = |g| for a fresh g ~ N(0, I_d), so cos(q_h, K) = 0.9 and |K| looks like a Gaussian row;
  * recency bump (long-context workload): for the last 512 positions, every key of KV group k gets
    + gamma * m_k with m_k the normalised sum of the group's unit queries and
    gamma = 2 sqrt(d) / min_g(q_g . m_k), which raises every head's logit there by at least 2 nats.

Workloads (sizes as used by the parity tests and the benchmark):
  1 tiny:    B1, H1/Hkv1, d64, nk1024, fp32, no spikes, i.i.d. S=16
  2 llama:   B1, H32/Hkv8, d128, nk32768, bf16, 32 spikes per head, stratified S=256
  3 batched: B8, H32/Hkv8, d128, nk32768, bf16, 32 spikes per head, systematic S in {64..1024}
  4 qwen:    B1, H28/Hkv4, d128, nk131072, bf16, 131 spikes per head (0.1%) + recency bump, strat S=512
  5 ternary: B4, H32/Hkv8, d128, nk65536, bf16, 32 spikes per head, ternary queries, strat S=256
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    d: int
    nk: int
    dtype: str                 # "bf16" or "f32"
    mode: str                  # "iid", "strat" or "sys"
    S: int
    ternary: bool
    seed: int                  # sampler seed
    q: torch.Tensor            # [B, H, d]          (CPU, dtype)
    K: torch.Tensor            # [B, nk, Hkv, d]    (CPU, dtype)
    V: torch.Tensor            # [B, nk, Hkv, d]    (CPU, dtype)
    S_sweep: list = field(default_factory=list)
    info: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.H // self.Hkv

    def numpy_inputs(self):
        """float32 numpy views of the exact input values (bf16 widens exactly to fp32)."""
        return (self.q.float().numpy(), self.K.float().numpy(), self.V.float().numpy())


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x)


def make_inputs(B: int, H: int, Hkv: int, d: int, nk: int, *, dtype: str = "bf16", spikes_per_head: int = 0,
                recency: int = 0, rng_seed: int = 0, q_scale: float = 1.0, k_scale: float = 1.0):
    """Gaussian q, K, V with optional planted spikes and recency bump; returns (q, K, V, info)."""
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    G = H // Hkv
    rng = np.random.Generator(np.random.PCG64(rng_seed))
    q = rng.standard_normal((B, H, d), dtype=np.float32) * np.float32(q_scale)
    K = rng.standard_normal((B, nk, Hkv, d), dtype=np.float32) * np.float32(k_scale)
    V = rng.standard_normal((B, nk, Hkv, d), dtype=np.float32)
    info = {"spikes_per_head": spikes_per_head, "recency": recency, "rng_seed": rng_seed}
    P = spikes_per_head
    if P:
        if G * P > nk:
            raise ValueError("too many spikes for nk")
        c_par, c_perp = 0.9, math.sqrt(1.0 - 0.81)
        for b in range(B):
            for kv in range(Hkv):
                pos = rng.choice(nk, size=G * P, replace=False)
                for g in range(G):
                    h = kv * G + g
                    qh = _unit(q[b, h].astype(np.float64))
                    for n in pos[g * P:(g + 1) * P]:
                        w = rng.standard_normal(d)
                        w -= (w @ qh) * qh
                        w = _unit(w)
                        r = np.linalg.norm(rng.standard_normal(d))
                        K[b, n, kv] = (r * (c_par * qh + c_perp * w)).astype(np.float32)
    if recency:
        for b in range(B):
            for kv in range(Hkv):
                qg = q[b, kv * G:(kv + 1) * G].astype(np.float64)
                m = _unit(np.sum(qg / np.linalg.norm(qg, axis=1, keepdims=True), axis=0))
                proj = qg @ m
                if proj.min() <= 0:
                    raise ValueError("recency bump needs every query of the group to project positively")
                gamma = 2.0 * math.sqrt(d) / proj.min()
                K[b, nk - recency:, kv] += (gamma * m).astype(np.float32)
    return _cast(q, dtype), _cast(K, dtype), _cast(V, dtype), info


CONFIGS = {
    1: dict(name="tiny", B=1, H=1, Hkv=1, d=64, nk=1024, dtype="f32", mode="iid", S=16, ternary=False,
            spikes=0, recency=0),
    2: dict(name="llama3.1-8b-32k", B=1, H=32, Hkv=8, d=128, nk=32768, dtype="bf16", mode="strat", S=256,
            ternary=False, spikes=32, recency=0),
    3: dict(name="batched-8x32k", B=8, H=32, Hkv=8, d=128, nk=32768, dtype="bf16", mode="sys", S=256,
            ternary=False, spikes=32, recency=0, S_sweep=[64, 128, 256, 512, 1024]),
    4: dict(name="qwen2.5-7b-128k", B=1, H=28, Hkv=4, d=128, nk=131072, dtype="bf16", mode="strat", S=512,
            ternary=False, spikes=131, recency=512),
    5: dict(name="ternary-4x64k", B=4, H=32, Hkv=8, d=128, nk=65536, dtype="bf16", mode="strat", S=256,
            ternary=True, spikes=32, recency=0),
}


def make(config: int, *, nk: int | None = None, B: int | None = None, S: int | None = None,
         spikes: int | None = None, seed: int = 1) -> Workload:
    """Workload `config` (1..5) with optional overrides of nk, batch, S and spikes per head.

    Input arrays use PCG64 seed 1000 + config; `seed` is the sampler seed.
    """
    c = dict(CONFIGS[config])
    if nk is not None:
        c["nk"] = nk
    if B is not None:
        c["B"] = B
    if S is not None:
        c["S"] = S
    if spikes is not None:
        c["spikes"] = spikes
    recency = min(c["recency"], c["nk"]) if c["recency"] else 0
    q, K, V, info = make_inputs(c["B"], c["H"], c["Hkv"], c["d"], c["nk"], dtype=c["dtype"],
                                spikes_per_head=c["spikes"], recency=recency, rng_seed=1000 + config)
    return Workload(name=c["name"], B=c["B"], H=c["H"], Hkv=c["Hkv"], d=c["d"], nk=c["nk"], dtype=c["dtype"],
                    mode=c["mode"], S=c["S"], ternary=c["ternary"], seed=seed, q=q, K=K, V=V,
                    S_sweep=list(c.get("S_sweep", [])), info=info)

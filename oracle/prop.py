"""Plain fp64 CPU oracle for S²ANTA-prop, the proportional-budget kernel family.

TEST INFRASTRUCTURE ONLY. This module is the checker, not the product: only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it. It shares no code
with the HIP path and imports nothing from it.

Source: "Stochastic Sparse Attention for Memory-Bound Inference", Section 3.2 and Appendix O:
  * pass 1 (Algorithm 3): the keys are cut into tiles of B_tile keys; per tile t and head h the tile
    max m_{h,t}, the exponentials u_{h,n} = exp(s_{h,n} - m_{h,t}) and their sum l_{h,t};
  * budgets (Algorithm 4): m* = max_t m_t, W_t = exp(m_t - m*) l_t, Z = sum_t W_t, q_t = S W_t / Z,
    S_t = floor(q_t), and the S - sum_t S_t samples left over go to the tiles with the largest fractional
    parts of q_t (largest remainder); invdelta_t = S_t / l_t (0 when S_t = 0); a0_t ~ U(0,1);
  * pass 2 (Algorithm 5): within tile t, with p running over the tile's keys in increasing order,
    x_n = invdelta_t u_n and c_n = floor(a0 + p + x_n) - floor(a0 + p), p <- p + x_n (systematic
    counts); the output is (1/S) sum_n c_n V_n (Algorithm 2, "return O/S").

Readings where the pages are silent (each is also listed in the design notes):
  * a0_{h,t} = U53(Philox4x32-10(counter (t, h, b, 3), key = seed)), the same generator and uniform as
    the other modes (tag 3 is otherwise unused);
  * ties between equal fractional parts go to the lower tile index; Z is a plain running sum over the
    tiles in order; the expression a0 + p + x is evaluated left to right;
  * the sampled indices are listed tile by tile, each key repeated c_n times (increasing key order).

parity unpinned: none of the functions below; see tests/test_oracle_prop.py for the pins.
"""

from __future__ import annotations

import math

import numpy as np

from . import philox
from .santa import DecodeResult, round_to_bf16, round_to_f32, scores_exact, scores_ternary

PROP = 3
TAG_PROP = 3
TILE = 256


def tile_stats(s: np.ndarray, tile: int):
    """Algorithm 3: per tile t the max m_t, the exponentials u_n = exp(s_n - m_t) and l_t = sum u."""
    s = np.asarray(s, dtype=np.float64)
    nk = s.shape[0]
    T = (nk + tile - 1) // tile
    m = np.empty(T)
    l = np.empty(T)
    u = np.empty(nk)
    for t in range(T):
        seg = s[t * tile:(t + 1) * tile]
        m[t] = np.max(seg)
        u[t * tile:(t + 1) * tile] = np.exp(seg - m[t])
        total = 0.0
        for v in u[t * tile:(t + 1) * tile]:
            total += v
        l[t] = total
    return m, u, l


def budgets(m: np.ndarray, l: np.ndarray, S: int):
    """Algorithm 4: integer tile budgets S_t summing to S, by largest remainder.

    Returns (S_t, q_t, W_t, Z).
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    m_star = float(np.max(m))
    W = np.exp(m - m_star) * l
    Z = 0.0
    for w in W:
        Z += w
    q = (float(S) * W) / Z
    St = np.floor(q).astype(np.int64)
    R = S - int(St.sum())
    if R < 0 or R > St.shape[0]:
        raise AssertionError(f"largest remainder: {R} samples left over for {St.shape[0]} tiles")
    frac = q - np.floor(q)
    order = sorted(range(St.shape[0]), key=lambda t: (-frac[t], t))
    for t in order[:R]:
        St[t] += 1
    return St, q, W, Z


def tile_counts(u: np.ndarray, l_t: float, S_t: int, a0: float):
    """Algorithm 5, its counting step: systematic counts of one tile's keys for budget S_t and offset a0.

    Returns (c, y): integer counts and the running values y_n = a0 + p after key n (y_{-1} = a0), whose
    distance to the nearest integer tells how close each count was to changing.
    """
    invdelta = (float(S_t) / l_t) if S_t > 0 else 0.0
    c = np.zeros(u.shape[0], dtype=np.int64)
    y = np.empty(u.shape[0] + 1)
    y[0] = a0
    p = 0.0
    for n, un in enumerate(np.asarray(u, dtype=np.float64)):
        x = invdelta * un
        c[n] = math.floor(a0 + p + x) - math.floor(a0 + p)
        p = p + x
        y[n + 1] = a0 + p
    return c, y


def offsets(seed: int, b: int, h: int, T: int) -> np.ndarray:
    """a0_{h,t} ~ U(0,1) per tile (Algorithm 4, the tile's random offset), from Philox counter (t, h, b, 3)."""
    return np.asarray(philox.uniforms(seed, np.arange(T, dtype=np.int64), h, b, TAG_PROP), dtype=np.float64)


def head_counts(s: np.ndarray, S: int, seed: int, b: int, h: int, tile: int = TILE):
    """Counts c_n over all keys of one head (Algorithms 3-5), plus the per-key boundary distances."""
    m, u, l = tile_stats(s, tile)
    St, _, _, _ = budgets(m, l, S)
    a0 = offsets(seed, b, h, m.shape[0])
    c = np.zeros(u.shape[0], dtype=np.int64)
    dist = np.zeros(u.shape[0])
    for t in range(m.shape[0]):
        sl = slice(t * tile, min((t + 1) * tile, u.shape[0]))
        ct, y = tile_counts(u[sl], l[t], int(St[t]), float(a0[t]))
        c[sl] = ct
        d = np.abs(y - np.round(y))
        dist[sl] = np.minimum(d[:-1], d[1:])
    return c, dist, St


def decode(q, K, V, S: int, seed: int, out_dtype: str = "bf16", ternary: bool = False, tile: int = TILE,
           keep_prob: bool = True, scores=None) -> DecodeResult:
    """One decode step of S²ANTA-prop. Same layouts as ``oracle.decode``; ``idx`` lists each head's
    sampled keys in increasing order with multiplicity (length S), ``delta`` the distance of the
    running value a0 + p to the nearest integer at either end of each sampled key (a count can only
    differ between two correct evaluations where that distance is at rounding level)."""
    q = np.asarray(q)
    K = np.asarray(K)
    V = np.asarray(V)
    B, H, d = q.shape
    _, nk, Hkv, _ = K.shape
    G = H // Hkv
    rnd = round_to_bf16 if out_dtype == "bf16" else round_to_f32
    est = np.zeros((B, H, d))
    idx = np.full((B, H, S), -1, dtype=np.int64)
    delta = np.zeros((B, H, S))
    counts = np.zeros((B, H, nk), dtype=np.int64)
    budget = np.zeros((B, H, (nk + tile - 1) // tile), dtype=np.int64)
    prob = np.zeros((B, H, nk)) if keep_prob else np.zeros((0,))
    unique = np.zeros((B, Hkv), dtype=np.int64)
    for b in range(B):
        for kv in range(Hkv):
            Kf = np.asarray(K[b, :, kv, :], dtype=np.float64)
            Vf = np.asarray(V[b, :, kv, :], dtype=np.float64)
            hit = np.zeros(nk, dtype=bool)
            for g in range(G):
                h = kv * G + g
                if scores is not None:
                    s = np.asarray(scores[b, h], dtype=np.float64)
                else:
                    s = scores_ternary(q[b, h], Kf, seed, b, h) if ternary else scores_exact(q[b, h], Kf)
                c, dist, St = head_counts(s, S, seed, b, h, tile)
                counts[b, h] = c
                budget[b, h] = St
                keys = np.repeat(np.arange(nk), c)[:S]
                idx[b, h, :keys.shape[0]] = keys
                delta[b, h, :keys.shape[0]] = np.repeat(dist, c)[:S]
                est[b, h] = (c.astype(np.float64) @ Vf) / float(S)
                hit |= c > 0
                if keep_prob:
                    e = np.exp(s - np.max(s))
                    prob[b, h] = e / np.sum(e)
            unique[b, kv] = int(hit.sum())
    res = DecodeResult(out=rnd(est), est=est, idx=idx, T=np.zeros((B, H, S)), delta=delta, prob=prob,
                       mu=np.zeros((B, H, d)), unique=unique, m_star=np.zeros((B, H)), Z=np.zeros((B, H)))
    res.extra["counts"] = counts
    res.extra["budgets"] = budget
    return res


def expected_estimate(s: np.ndarray, Vmat: np.ndarray, S: int, tile: int = TILE) -> np.ndarray:
    """E over the offsets a0 of the prop estimate of one head: (1/S) sum_t S_t sum_{n in t} (u_n/l_t) V_n
    (each systematic count has mean x_n = S_t u_n / l_t)."""
    m, u, l = tile_stats(s, tile)
    St, _, _, _ = budgets(m, l, S)
    w = np.zeros(u.shape[0])
    for t in range(m.shape[0]):
        sl = slice(t * tile, min((t + 1) * tile, u.shape[0]))
        w[sl] = St[t] * u[sl] / l[t]
    return (w @ np.asarray(Vmat, dtype=np.float64)) / float(S)

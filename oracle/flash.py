"""Plain fp64 CPU oracle for S²ANTA-flash, the speculative per-tile kernel family.

TEST INFRASTRUCTURE ONLY. This module is the checker, not the product: only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it. It shares no code
with the HIP path and imports nothing from it.

Source: "Stochastic Sparse Attention for Memory-Bound Inference", Section 3.3 and Appendix P
(Algorithms 6-8):
  * kernel 1, per tile t of B_tile keys and head h: scores, the tile max m_{h,t}, u_{h,n} = exp(s_{h,n} -
    m_{h,t}) and l_{h,t} = sum u; every tile gets the same budget S_tile ~ S / T; invdelta = S_tile / l_{h,t},
    a0 ~ U(0,1); systematic counts c_n = floor(a0 + p + x_n) - floor(a0 + p) with x_n = invdelta u_n (the
    same in-tile rule as S²ANTA-prop's pass 2), and the tile partial Otilde_{h,t} = sum_n c_n V_n;
  * kernel 2, per head: m* = max_t m_t, W_t = exp(m_t - m*) l_t, Z = sum_t W_t and
    O_h = (1/Z) sum_t W_t Otilde_{h,t} / S_tile.

Readings where the pages are silent (each is also listed in the design notes):
  * S_tile = max(1, round(S / T)) with halves rounded up, i.e. floor((2 S + T) / (2 T)), at least 1;
  * a0_{h,t} = U53(Philox4x32-10(counter (t, h, b, 4), key = seed)), tag 4 being otherwise unused;
  * each head lists T * S_tile sampled keys: tile t's in slots [t S_tile, (t+1) S_tile), in increasing key
    order with multiplicity;
  * Z is a running sum over the tiles in order, and the merge adds W_t * Otilde_t over t in order before
    dividing by Z * S_tile.

parity unpinned: none of the functions below; see tests/test_oracle_flash.py for the pins.
"""

from __future__ import annotations

import numpy as np

from . import philox
from .prop import tile_counts, tile_stats
from .santa import DecodeResult, round_to_bf16, round_to_f32, scores_exact, scores_ternary

FLASH = 4
TAG_FLASH = 4
TILE = 256


def tile_budget(S: int, T: int) -> int:
    """Algorithm 6, its budget step: the uniform per-tile budget S_tile ~ S / T, rounded half up, at least 1."""
    return max(1, (2 * S + T) // (2 * T))


def offsets(seed: int, b: int, h: int, T: int) -> np.ndarray:
    """a0_{h,t} ~ U(0,1) per tile (Algorithm 7, the tile's random offset), from Philox counter (t, h, b, 4)."""
    return np.asarray(philox.uniforms(seed, np.arange(T, dtype=np.int64), h, b, TAG_FLASH), dtype=np.float64)


def merge_weights(m: np.ndarray, l: np.ndarray):
    """Algorithm 8, its reweighting step: W_t = exp(m_t - m*) l_t and Z = sum_t W_t (in tile order)."""
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    W = np.exp(m - float(np.max(m))) * l
    Z = 0.0
    for w in W:
        Z += w
    return W, Z


def head_estimate(s: np.ndarray, Vmat: np.ndarray, S: int, a0: np.ndarray, tile: int = TILE):
    """One head: (estimate, counts, boundary distances, S_tile, W, Z) for per-tile offsets a0."""
    m, u, l = tile_stats(s, tile)
    T = m.shape[0]
    st = tile_budget(S, T)
    Vmat = np.asarray(Vmat, dtype=np.float64)
    c = np.zeros(u.shape[0], dtype=np.int64)
    dist = np.zeros(u.shape[0])
    parts = np.zeros((T, Vmat.shape[1]))
    for t in range(T):
        sl = slice(t * tile, min((t + 1) * tile, u.shape[0]))
        ct, y = tile_counts(u[sl], l[t], st, float(a0[t]))
        c[sl] = ct
        d = np.abs(y - np.round(y))
        dist[sl] = np.minimum(d[:-1], d[1:])
        parts[t] = ct.astype(np.float64) @ Vmat[sl]
    W, Z = merge_weights(m, l)
    acc = np.zeros(Vmat.shape[1])
    for t in range(T):
        acc = acc + W[t] * parts[t]
    return acc / (Z * st), c, dist, st, W, Z


def decode(q, K, V, S: int, seed: int, out_dtype: str = "bf16", ternary: bool = False, tile: int = TILE,
           keep_prob: bool = True, scores=None) -> DecodeResult:
    """One decode step of S²ANTA-flash. Same layouts as ``oracle.decode``; ``idx`` has T * S_tile entries
    per head (tile-major, increasing key order with multiplicity inside a tile), ``delta`` the distance of
    the running value a0 + p to the nearest integer at either end of each sampled key."""
    q = np.asarray(q)
    K = np.asarray(K)
    V = np.asarray(V)
    B, H, d = q.shape
    _, nk, Hkv, _ = K.shape
    G = H // Hkv
    T = (nk + tile - 1) // tile
    st = tile_budget(S, T)
    L = T * st
    rnd = round_to_bf16 if out_dtype == "bf16" else round_to_f32
    est = np.zeros((B, H, d))
    idx = np.full((B, H, L), -1, dtype=np.int64)
    delta = np.zeros((B, H, L))
    counts = np.zeros((B, H, nk), dtype=np.int64)
    weights = np.zeros((B, H, T))
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
                a0 = offsets(seed, b, h, T)
                e, c, dist, _, W, Z = head_estimate(s, Vf, S, a0, tile)
                est[b, h] = e
                counts[b, h] = c
                weights[b, h] = W / Z
                for t in range(T):
                    lo, hi = t * tile, min((t + 1) * tile, nk)
                    keys = np.repeat(np.arange(lo, hi), c[lo:hi])
                    idx[b, h, t * st:t * st + keys.shape[0]] = keys
                    delta[b, h, t * st:t * st + keys.shape[0]] = np.repeat(dist[lo:hi], c[lo:hi])
                hit |= c > 0
                if keep_prob:
                    ex = np.exp(s - np.max(s))
                    prob[b, h] = ex / np.sum(ex)
            unique[b, kv] = int(hit.sum())
    res = DecodeResult(out=rnd(est), est=est, idx=idx, T=np.zeros((B, H, L)), delta=delta, prob=prob,
                       mu=np.zeros((B, H, d)), unique=unique, m_star=np.zeros((B, H)), Z=np.zeros((B, H)))
    res.extra["counts"] = counts
    res.extra["weights"] = weights
    res.extra["S_tile"] = st
    return res


def estimate_from_idx(Vmat: np.ndarray, idx: np.ndarray, weights: np.ndarray, S_tile: int, tile: int = TILE):
    """The flash estimate for a given index list (T * S_tile entries, tile-major) and merge weights W_t / Z:
    sum_t (W_t / Z) * (sum of the tile's listed rows) / S_tile."""
    Vmat = np.asarray(Vmat, dtype=np.float64)
    acc = np.zeros(Vmat.shape[1])
    T = weights.shape[0]
    for t in range(T):
        rows = idx[t * S_tile:(t + 1) * S_tile]
        rows = rows[rows >= 0]
        acc = acc + weights[t] * Vmat[rows].sum(axis=0)
    return acc / S_tile

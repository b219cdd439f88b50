"""Plain fp64 CPU oracle for one decode step of SANTA / S²ANTA attention.

TEST INFRASTRUCTURE ONLY. This module is the checker, not the product: only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it. It shares no code
with the HIP path and imports nothing from it.

Source: "Stochastic Sparse Attention for Memory-Bound Inference" (Lee et al., arXiv:2605.01910):
  * scaled dot-product attention for one decode query, Attn(q,K,V) = softmax(qK^T/sqrt(dk)) V = AV
    (Section 2, Eq. 1);
  * SANTA: S indices drawn i.i.d. from the post-softmax categorical A, output = mean of the S gathered
    V rows (Section 2, Eq. 4; Appendix A, Eq. 7 and Definition A.1);
  * S²ANTA-strat / S²ANTA-sys: equal-mass strata I_m = [m/S, (m+1)/S), one point per stratum, either
    independent (strat) or one shared offset (sys), mapped through the inverse CDF (Section 2.1,
    "Construction"); the inverse-CDF convention is the indicator 1{F(j-1) <= t < F(j)} used in the proof
    of Proposition A.4 (Appendix A.4);
  * Bernoulli ternary query for the score stage (Section 5, Eq. 5; Appendix C, Eqs. 8-9);
  * GQA: query head h reads KV head floor(h/G), G = H/Hkv (Appendix O, Algorithm 2).

Everything is computed in float64 on the exact values of the (bf16- or fp32-cast) inputs. The random
numbers come from ``oracle.philox`` (counter-based, keyed by seed, batch, head and sample index).

Readings where the pages are silent (each is also listed in the design notes):
  * scale c = 1/sqrt(d) formed in fp64 and applied after the dot product;
  * systematic points T_m = (m + u)/S with one u ~ U[0,1), i.e. U = u/S ~ U[0, 1/S), T_m = U + m/S;
    stratified points T_m = (m + u_m)/S; i.i.d. points T_m = u_m;
  * a point at or beyond F_nk because of rounding takes the last key with nonzero probability;
  * ternary mode uses one Bernoulli sample (B = 1) and norm = max_i |q_i| per (batch, head); a query that
    is all zero scores every key 0; sign(0) = 0; the Bernoulli test is u < |q_i|/norm;
  * outputs are rounded to the input dtype, round-to-nearest-even.

parity unpinned: none of the functions below; see tests/test_oracle_*.py for the pins.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import philox

IID, STRAT, SYS = 0, 1, 2
TERNARY_Q = 0x100
MODE_NAMES = {IID: "iid", STRAT: "strat", SYS: "sys"}


# ---------------------------------------------------------------------------------------------
# numeric helpers


def scale(d: int) -> float:
    """Softmax temperature 1/sqrt(dk) (Section 2, Eq. 1), formed in fp64."""
    return 1.0 / math.sqrt(d)


def round_to_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (8 significant bits), ties to even.

    Direct from fp64 (no intermediate fp32 rounding). Values below the bf16 normal range are not
    expected here and are rounded as if the exponent range were unbounded.
    """
    x = np.asarray(x, dtype=np.float64)
    mant, expo = np.frexp(x)  # x = mant * 2**expo, 0.5 <= |mant| < 1
    return np.ldexp(np.round(np.ldexp(mant, 8)), expo - 8)  # np.round is half-to-even


def round_to_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------------------------
# score stage


def scores_exact(qrow: np.ndarray, Kmat: np.ndarray) -> np.ndarray:
    """s_n = (q . K_n) / sqrt(dk) for one query head over all nk keys (Section 2, Eq. 1)."""
    qrow = np.asarray(qrow, dtype=np.float64)
    Kmat = np.asarray(Kmat, dtype=np.float64)
    return (Kmat @ qrow) * scale(qrow.shape[0])


def ternary_query(qrow: np.ndarray, seed: int, b: int, h: int, n: int = 0):
    """Bernoulli ternary query (Section 5, Eq. 5; Appendix C, Eqs. 8-9).

    q is normalised by norm = max_i |q_i| so every |q_i|/norm is a probability; each element becomes
    sign(q_i) * Bernoulli(|q_i|/norm) in {-1, 0, +1}. Returns (qhat, norm).
    """
    qrow = np.asarray(qrow, dtype=np.float64)
    norm = float(np.max(np.abs(qrow))) if qrow.size else 0.0
    if norm == 0.0:
        return np.zeros_like(qrow), 0.0
    prob = np.abs(qrow) / norm
    u = philox.uniforms(seed, np.arange(qrow.shape[0]), h, b, philox.TAG_BERNOULLI + 256 * n)
    qhat = np.where(u < prob, np.sign(qrow), 0.0)
    return qhat, norm


def scores_ternary(qrow: np.ndarray, Kmat: np.ndarray, seed: int, b: int, h: int) -> np.ndarray:
    """Unbiased score estimate p_hat = norm * qhat K^T, then the 1/sqrt(dk) scale (Eq. 5 with B = 1)."""
    qhat, norm = ternary_query(qrow, seed, b, h)
    Kmat = np.asarray(Kmat, dtype=np.float64)
    return ((Kmat @ qhat) * norm) * scale(qhat.shape[0])


# ---------------------------------------------------------------------------------------------
# softmax, CDF, sampling


def softmax(s: np.ndarray):
    """A = softmax(s): returns (p, m_star, Z) with p_n = exp(s_n - m*)/Z (Section 2, Eq. 1)."""
    s = np.asarray(s, dtype=np.float64)
    m_star = float(np.max(s))
    e = np.exp(s - m_star)
    Z = float(np.sum(e))
    return e / Z, m_star, Z


def cdf(p: np.ndarray) -> np.ndarray:
    """F_n = sum_{j<=n} p_j, a plain sequential running sum (Section 2.1, 'Construction')."""
    return np.cumsum(np.asarray(p, dtype=np.float64))


def sample_points(mode: int, S: int, seed: int, b: int, h: int) -> np.ndarray:
    """The S points T_m in [0,1) that the inverse CDF maps to key indices.

    IID (SANTA, Section 2 and Definition A.1): T_m ~ U[0,1) independently.
    STRAT (S²ANTA-strat, Section 2.1): T_m ~ U(I_m), I_m = [m/S, (m+1)/S), independent across m.
    SYS (S²ANTA-sys, Section 2.1): one U ~ U[0, 1/S), T_m = U + m/S.
    """
    m = np.arange(S, dtype=np.int64)
    if mode == IID:
        return philox.uniforms(seed, m, h, b, philox.TAG_POINT)
    if mode == STRAT:
        u = philox.uniforms(seed, m, h, b, philox.TAG_POINT)
        return (m.astype(np.float64) + u) / float(S)
    if mode == SYS:
        u = philox.uniforms(seed, 0, h, b, philox.TAG_SYS)
        return (m.astype(np.float64) + float(u)) / float(S)
    raise ValueError(f"unknown sampling mode {mode}")


def inverse_cdf(F: np.ndarray, p: np.ndarray, T: np.ndarray):
    """J_m = the key j with F(j-1) <= T_m < F(j) (Appendix A.4, the indicator in the proof of
    Proposition A.4). Zero-mass keys are never chosen. A point at or beyond F_nk (rounding) takes the
    last key with p > 0.

    Returns (J, delta): 0-based key indices and each point's distance to the nearer edge of its
    interval [F(J-1), F(J)).
    """
    F = np.asarray(F, dtype=np.float64)
    T = np.asarray(T, dtype=np.float64)
    nk = F.shape[0]
    J = np.searchsorted(F, T, side="right")
    over = J >= nk
    if np.any(over):
        J = J.copy()
        J[over] = int(np.nonzero(np.asarray(p) > 0)[0][-1])
    lo = np.where(J > 0, F[np.maximum(J - 1, 0)], 0.0)
    hi = F[J]
    delta = np.minimum(np.abs(T - lo), np.abs(hi - T))
    return J.astype(np.int64), delta


def estimate(Vmat: np.ndarray, J: np.ndarray, S: int) -> np.ndarray:
    """(1/S) sum_m V_{J_m}: gather-and-add of the sampled rows (Section 2, Eq. 4; Appendix A, Eq. 7)."""
    Vmat = np.asarray(Vmat)
    return np.asarray(Vmat[np.asarray(J)], dtype=np.float64).sum(axis=0) / float(S)


# ---------------------------------------------------------------------------------------------
# whole decode step


@dataclass
class DecodeResult:
    out: np.ndarray          # [B,H,d] estimator rounded to the output dtype (as float64)
    est: np.ndarray          # [B,H,d] estimator in fp64 before rounding
    idx: np.ndarray          # [B,H,S] sampled key indices (int64)
    T: np.ndarray            # [B,H,S] sample points
    delta: np.ndarray        # [B,H,S] distance of each point to its interval's nearer edge
    prob: np.ndarray         # [B,H,nk] softmax probabilities
    mu: np.ndarray           # [B,H,d] dense attention output AV (fp64)
    unique: np.ndarray       # [B,Hkv] number of distinct V rows the G heads of a group sample
    m_star: np.ndarray       # [B,H]
    Z: np.ndarray            # [B,H]
    extra: dict = field(default_factory=dict)


def decode(q, K, V, S: int, mode: int, seed: int, out_dtype: str = "bf16", ternary: bool = False,
           keep_prob: bool = True, scores=None) -> DecodeResult:
    """One decode step of SANTA (mode IID) or S²ANTA (STRAT / SYS), with exact or ternary scores.

    q: [B, H, d]; K, V: [B, nk, Hkv, d] (sequence-major cache, Appendix Q); any float dtype holding the
    exact input values. Query head h reads KV head h // (H/Hkv) (Appendix O, Algorithm 2).
    """
    q = np.asarray(q)
    K = np.asarray(K)
    V = np.asarray(V)
    B, H, d = q.shape
    _, nk, Hkv, _ = K.shape
    if H % Hkv:
        raise ValueError("heads must be a multiple of kv_heads")
    G = H // Hkv
    rnd = round_to_bf16 if out_dtype == "bf16" else round_to_f32
    est = np.zeros((B, H, d))
    mu = np.zeros((B, H, d))
    idx = np.zeros((B, H, S), dtype=np.int64)
    T = np.zeros((B, H, S))
    delta = np.zeros((B, H, S))
    prob = np.zeros((B, H, nk)) if keep_prob else np.zeros((0,))
    unique = np.zeros((B, Hkv), dtype=np.int64)
    m_star = np.zeros((B, H))
    Z = np.zeros((B, H))
    for b in range(B):
        for kv in range(Hkv):
            Kf = np.asarray(K[b, :, kv, :], dtype=np.float64)
            Vf = np.asarray(V[b, :, kv, :], dtype=np.float64)
            group = []
            for g in range(G):
                h = kv * G + g
                if scores is not None:
                    s = np.asarray(scores[b, h], dtype=np.float64)
                elif ternary:
                    s = scores_ternary(q[b, h], Kf, seed, b, h)
                else:
                    s = scores_exact(q[b, h], Kf)
                p, m_star[b, h], Z[b, h] = softmax(s)
                F = cdf(p)
                T[b, h] = sample_points(mode, S, seed, b, h)
                idx[b, h], delta[b, h] = inverse_cdf(F, p, T[b, h])
                est[b, h] = estimate(Vf, idx[b, h], S)
                mu[b, h] = p @ Vf
                if keep_prob:
                    prob[b, h] = p
                group.append(idx[b, h])
            unique[b, kv] = np.unique(np.concatenate(group)).size
    return DecodeResult(out=rnd(est), est=est, idx=idx, T=T, delta=delta, prob=prob, mu=mu,
                        unique=unique, m_star=m_star, Z=Z)


def dense(q, K, V, out_dtype: str = "bf16"):
    """Dense decode attention softmax(qK^T/sqrt(dk))V per query head (Section 2, Eq. 1), fp64.

    Returns (mu_fp64, mu_rounded).
    """
    q = np.asarray(q)
    K = np.asarray(K)
    V = np.asarray(V)
    B, H, d = q.shape
    _, nk, Hkv, _ = K.shape
    G = H // Hkv
    mu = np.zeros((B, H, d))
    for b in range(B):
        for kv in range(Hkv):
            Kf = np.asarray(K[b, :, kv, :], dtype=np.float64)
            Vf = np.asarray(V[b, :, kv, :], dtype=np.float64)
            for g in range(G):
                h = kv * G + g
                p, _, _ = softmax(scores_exact(q[b, h], Kf))
                mu[b, h] = p @ Vf
    rnd = round_to_bf16 if out_dtype == "bf16" else round_to_f32
    return mu, rnd(mu)


# ---------------------------------------------------------------------------------------------
# accounting and variance closed forms


def bytes_touched(B: int, nk: int, H: int, Hkv: int, d: int, elt: int, unique_total: int) -> dict:
    """Bytes a decode step must move: all of K, the distinct sampled V rows, q and out.

    The value-stage reads follow Appendix E, Table 8 (S·dk reads per query instead of nk·dk), with the
    rows shared by the G heads of a KV group counted once (Appendix O, Algorithm 5, emitted-row set).
    """
    bk = B * nk * Hkv * d * elt
    bv = unique_total * d * elt
    bqo = 2 * B * H * d * elt
    return {"bytes_k": bk, "bytes_v": bv, "bytes_qo": bqo, "bytes_total": bk + bv + bqo}


def var_trace_iid(p: np.ndarray, Vmat: np.ndarray, S: int) -> float:
    """tr Cov(SANTA estimate) = tr(Sigma)/S, tr(Sigma) = sum_j p_j ||V_j||^2 - ||mu||^2
    (Proposition A.3; Appendix M, multinomial closed form)."""
    p = np.asarray(p, dtype=np.float64)
    Vmat = np.asarray(Vmat, dtype=np.float64)
    mu = p @ Vmat
    return float((p @ np.sum(Vmat * Vmat, axis=1) - mu @ mu) / S)


def stratum_weights(F: np.ndarray, m: int, S: int):
    """Distribution of J given T ~ U[m/S, (m+1)/S): the overlap of that stratum with each key's
    interval [F(j-1), F(j)), times S. Returns (keys, weights)."""
    F = np.asarray(F, dtype=np.float64)
    lo_t, hi_t = m / S, (m + 1) / S
    Fprev = np.concatenate(([0.0], F[:-1]))
    a = np.maximum(Fprev, lo_t)
    bnd = np.minimum(F, hi_t)
    w = np.clip(bnd - a, 0.0, None) * S
    keys = np.nonzero(w > 0)[0]
    return keys, w[keys]


def var_trace_strat(F: np.ndarray, Vmat: np.ndarray, S: int) -> float:
    """tr Cov(S²ANTA-strat estimate) = (1/S^2) sum_m tr(Sigma_m) (Appendix M, independent equal-mass
    stratified closed form; Theorem A.6)."""
    Vmat = np.asarray(Vmat, dtype=np.float64)
    total = 0.0
    for m in range(S):
        keys, w = stratum_weights(F, m, S)
        w = w / w.sum()
        Vk = Vmat[keys]
        mu_m = w @ Vk
        total += float(w @ np.sum(Vk * Vk, axis=1) - mu_m @ mu_m)
    return total / (S * S)

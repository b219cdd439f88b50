"""Plain fp64 CPU oracle for the mean-group-query Bernoulli score estimator.

TEST INFRASTRUCTURE ONLY. This module is the checker, not the product: only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it. It shares no code
with the HIP path and imports nothing from it.

Source: "Stochastic Sparse Attention for Memory-Bound Inference", Section 5.1 (Eq. 6) and Appendix C.2
(Eqs. 10-13):
  * the queries of a GQA group share one representative, the mean of their absolute values,
    m_i = (1/|G|) sum_g |q_{g,i}| (Eq. 10);
  * m is normalised by norm >= max_i m_i and estimated by B Bernoulli samples,
    mhat_i = (norm / B) sum_n b_i^(n), b_i^(n) ~ Bernoulli(m_i / norm) (Eqs. 11-12);
  * each query's scores are estimated as phat_g = (mhat ⊙ q_g / m)^T K (Eqs. 6 and 13), which only needs
    the key features i with mhat_i != 0: with a feature-major K^T those are whole rows left unread.

Readings where the pages are silent (each is also listed in the design notes):
  * norm = max_i m_i, the smallest allowed value;
  * the B samples are stratified per feature (Appendix C.1 says stratified Bernoulli sampling is used for
    B > 1): b_i^(n) = 1 iff (n + U_{i,n}) / B < m_i / norm, so c_i = sum_n b_i^(n) is floor or ceil of
    B m_i / norm; U_{i,n} = U53(Philox4x32-10(counter (i, kv, b, 5 + 256 n), key = seed));
  * the weight of feature i for query g is w_{g,i} = ((norm * c_i) / B) / m_i * q_{g,i} (left to right, 0
    where m_i = 0, i.e. where every query of the group is 0), and s_{g,n} = (sum_i w_{g,i} K_{n,i}) / sqrt(d_k);
  * m_i = (sum over g in order of |q_{g,i}|) / |G| in fp64; the comparisons deciding c_i are taken in fp64.

parity unpinned: none of the functions below; see tests/test_oracle_group_bernoulli.py for the pins.
"""

from __future__ import annotations

import numpy as np

from . import philox
from .santa import scale

TAG_GROUP = 5


def mean_group_query(qg: np.ndarray) -> np.ndarray:
    """Eq. 10: m_i = (1/|G|) sum_g |q_{g,i}| over the group's queries (rows of qg), summed in row order."""
    qg = np.asarray(qg, dtype=np.float64)
    acc = np.zeros(qg.shape[1])
    for row in qg:
        acc = acc + np.abs(row)
    return acc / float(qg.shape[0])


def uniforms(seed: int, b: int, kv: int, d: int, B: int) -> np.ndarray:
    """U_{i,n} for features i < d and samples n < B, shape [B, d]: Philox counter (i, kv, b, 5 + 256 n)."""
    return np.stack([np.asarray(philox.uniforms(seed, np.arange(d), kv, b, TAG_GROUP + 256 * n), dtype=np.float64)
                     for n in range(B)])


def stratified_counts(pi: np.ndarray, U: np.ndarray) -> np.ndarray:
    """Eqs. 11-12 with stratified samples: c_i = #{n < B : (n + U_{n,i}) / B < pi_i}."""
    pi = np.asarray(pi, dtype=np.float64)
    B = U.shape[0]
    c = np.zeros(pi.shape[0], dtype=np.int64)
    for n in range(B):
        c += ((float(n) + U[n]) / float(B) < pi).astype(np.int64)
    return c


def weights(qg: np.ndarray, m: np.ndarray, c: np.ndarray, norm: float, B: int) -> np.ndarray:
    """Eq. 13: w_{g,i} = (mhat_i / m_i) q_{g,i} with mhat_i = norm c_i / B; 0 where m_i = 0."""
    qg = np.asarray(qg, dtype=np.float64)
    mh = (norm * c.astype(np.float64)) / float(B)
    safe = np.where(m > 0.0, m, 1.0)
    ratio = np.where(m > 0.0, mh / safe, 0.0)
    return ratio[None, :] * qg


def group_scores(qg: np.ndarray, Kmat: np.ndarray, B: int, seed: int, b: int, kv: int):
    """Scores of every query of one KV group (rows of qg) against Kmat [nk, d]; returns (s [G, nk], c, norm)."""
    qg = np.asarray(qg, dtype=np.float64)
    d = qg.shape[1]
    m = mean_group_query(qg)
    norm = float(np.max(m))
    if norm == 0.0:
        return np.zeros((qg.shape[0], Kmat.shape[0])), np.zeros(d, dtype=np.int64), 0.0
    c = stratified_counts(m / norm, uniforms(seed, b, kv, d, B))
    w = weights(qg, m, c, norm, B)
    Kmat = np.asarray(Kmat, dtype=np.float64)
    return (w @ Kmat.T) * scale(d), c, norm


def scores(q, K, B: int, seed: int):
    """Scores [batch, heads, nk] of a whole decode step (K sequence-major [batch, nk, Hkv, d]) plus the
    per-group feature counts [batch, Hkv, d]."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K)
    Bt, H, d = q.shape
    _, nk, Hkv, _ = K.shape
    G = H // Hkv
    out = np.zeros((Bt, H, nk))
    counts = np.zeros((Bt, Hkv, d), dtype=np.int64)
    for b in range(Bt):
        for kv in range(Hkv):
            s, c, _ = group_scores(q[b, kv * G:(kv + 1) * G], K[b, :, kv, :], B, seed, b, kv)
            out[b, kv * G:(kv + 1) * G] = s
            counts[b, kv] = c
    return out, counts

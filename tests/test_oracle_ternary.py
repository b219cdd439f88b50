"""Pins for the oracle's Bernoulli ternary-query score estimate.

"Stochastic Sparse Attention for Memory-Bound Inference", Section 5 (Eq. 5) and Appendix C (Eqs. 8-9,
Section C.1, Figure 6). With q normalised by norm >= max|q_i|, each element is sign(q_i) with
probability |q_i|/norm and 0 otherwise; norm * qhat K^T is unbiased for q K^T (linearity), and the
variance of one key's estimate is sum_i K_i^2 (norm |q_i| - q_i^2) per Bernoulli sample.
"""

import json
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def test_ternary_values_and_signs():
    rng = np.random.default_rng(0)
    q = rng.standard_normal(128)
    for seed in range(50):
        qhat, norm = oracle.ternary_query(q, seed, 1, 3)
        assert norm == np.max(np.abs(q))
        assert set(np.unique(qhat)).issubset({-1.0, 0.0, 1.0})
        nz = qhat != 0
        assert np.all(np.sign(q[nz]) == qhat[nz])
        assert qhat[np.argmax(np.abs(q))] == np.sign(q[np.argmax(np.abs(q))])  # probability 1


def test_ternary_zero_query():
    qhat, norm = oracle.ternary_query(np.zeros(64), 5, 0, 0)
    assert norm == 0.0 and not np.any(qhat)
    s = oracle.scores_ternary(np.zeros(64), np.ones((10, 64)), 5, 0, 0)
    assert np.array_equal(s, np.zeros(10))


def test_bernoulli_keep_frequency():
    rng = np.random.default_rng(1)
    q = rng.standard_normal(64)
    n = 6000
    kept = np.zeros(64)
    for seed in range(n):
        kept += oracle.ternary_query(q, seed, 0, 7)[0] != 0
    prob = np.abs(q) / np.abs(q).max()
    sd = np.sqrt(prob * (1 - prob) / n)
    assert np.all(np.abs(kept / n - prob) <= 4.5 * sd + 1e-12)


def test_ternary_scores_unbiased_with_closed_form_variance():
    rng = np.random.default_rng(2)
    d, nk, n = 128, 48, 4096
    q = rng.standard_normal(d)
    K = rng.standard_normal((nk, d))
    exact = oracle.scores_exact(q, K)
    acc = np.zeros(nk)
    acc2 = np.zeros(nk)
    for seed in range(n):
        s = oracle.scores_ternary(q, K, seed, 2, 9)
        acc += s
        acc2 += s * s
    mean = acc / n
    norm = np.abs(q).max()
    c = oracle.scale(d)
    var = c * c * (K * K) @ (norm * np.abs(q) - q * q)
    z = np.abs(mean - exact) / np.sqrt(var / n)
    assert np.sum(z > 3) <= 2 and z.max() < 4.5
    emp = acc2 / n - mean * mean
    assert np.allclose(emp.mean() / var.mean(), 1.0, atol=0.06)


def test_figure6_error_level_B4():
    """Figure 6: B = 4 i.i.d. Bernoulli samples give about 60% mean relative L2 error (dk=128, nk=1024)."""
    g = json.load(open(os.path.join(HERE, "golden", "fig6_bernoulli.json")))
    rng = np.random.default_rng(6)
    dk, nk, inst, B = g["dk"], g["nk"], g["instances"], g["B"]
    errs = []
    for i in range(inst):
        q = rng.standard_normal(dk)
        K = rng.standard_normal((nk, dk)) / np.sqrt(dk)
        p = K @ q
        acc = np.zeros(dk)
        for n in range(B):
            qhat, norm = oracle.ternary_query(q, 1000 + i, 0, 0, n=n)
            acc += qhat
        phat = (norm / B) * (K @ acc)
        errs.append(np.linalg.norm(phat - p) / np.linalg.norm(p))
    level = float(np.mean(errs))
    assert abs(level - g["standard_rel_l2"]) < 0.08


def test_figure6_stratified_level_B4():
    """Figure 6 and Appendix C.1: stratified Bernoulli sampling at B = 4 gives about 30% mean relative L2
    error of the score estimate (dk=128, nk=1024). The stratified estimator is the mean-group-query one
    with a group of a single query (m = |q|, norm = max|q|, per-feature stratified counts)."""
    g = json.load(open(os.path.join(HERE, "golden", "fig6_bernoulli.json")))
    rng = np.random.default_rng(7)
    dk, nk, inst, B = g["dk"], g["nk"], g["instances"], g["B"]
    errs = []
    for i in range(inst):
        q = rng.standard_normal(dk)
        K = rng.standard_normal((nk, dk)) / np.sqrt(dk)
        exact = (K @ q) * oracle.scale(dk)
        s, c, norm = oracle.group_bernoulli.group_scores(q[None, :], K, B, 2000 + i, 0, 0)
        assert norm == np.max(np.abs(q)) and c.min() >= 0 and c.max() <= B
        errs.append(np.linalg.norm(s[0] - exact) / np.linalg.norm(exact))
    level = float(np.mean(errs))
    assert abs(level - g["stratified_rel_l2"]) < 0.08, level
    # and stratification halves the i.i.d. level the same figure prints
    assert level < 0.75 * g["standard_rel_l2"]

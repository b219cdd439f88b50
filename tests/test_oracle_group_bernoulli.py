"""Pins of the mean-group-query Bernoulli oracle (Section 5.1, Eq. 6; Appendix C.2, Eqs. 10-13) against
what the pages and the mathematics fix: the stratified counts' range and exact mean, the reduction to
the per-head ternary estimator (Eq. 5, itself pinned) for a one-query group with B = 1, unbiasedness of
the group score estimate, the O(1/B^2) variance of stratified sampling, and the generator."""

import math

import numpy as np
import pytest

import oracle
from oracle import group_bernoulli as gb
from oracle import philox


def test_mean_group_query_is_mean_of_absolute_values():
    qg = np.array([[1.0, -2.0, 0.0, 0.5], [-3.0, 2.0, 0.0, -0.5]])
    np.testing.assert_array_equal(gb.mean_group_query(qg), [2.0, 2.0, 0.0, 0.5])


@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_stratified_counts_range_and_exact_mean(B):
    """Each count is floor or ceil of B * pi; over U on a midpoint grid (the same U in every stratum) the
    mean count is B * pi exactly up to the grid's resolution: sum_n clamp(B pi - n, 0, 1) = B pi."""
    pi = np.linspace(0.0, 1.0, 41)
    rng = np.random.default_rng(B)
    for _ in range(20):
        c = gb.stratified_counts(pi, rng.uniform(0, 1, (B, pi.shape[0])))
        assert np.all((c == np.floor(B * pi)) | (c == np.ceil(B * pi)))
    N = 4000
    acc = np.zeros(pi.shape[0])
    for k in range(N):
        acc += gb.stratified_counts(pi, np.full((B, pi.shape[0]), (k + 0.5) / N))
    np.testing.assert_allclose(acc / N, B * pi, atol=B / N + 1e-12)


def test_single_query_B1_is_the_ternary_estimator():
    """|G| = 1, B = 1: m = |q|, c_i = [U_i < |q_i| / max|q|], w_i = norm c_i sign(q_i): the group estimate is
    norm * qhat K^T with the ternary query of Eq. 5 drawn from the same uniforms."""
    rng = np.random.default_rng(3)
    d, nk = 32, 50
    q = rng.normal(size=d)
    K = rng.normal(size=(nk, d))
    U = rng.uniform(0, 1, (1, d))
    m = gb.mean_group_query(q[None])
    norm = float(m.max())
    c = gb.stratified_counts(m / norm, U)
    w = gb.weights(q[None], m, c, norm, 1)
    qhat = np.where(U[0] < np.abs(q) / norm, np.sign(q), 0.0)
    np.testing.assert_allclose(w[0], norm * qhat, rtol=1e-15)
    # the oracle's own ternary estimator uses the same rule (Eq. 9) on its Philox uniforms
    qh2, n2 = oracle.ternary_query(q, 7, 0, 1)
    u2 = philox.uniforms(7, np.arange(d), 1, 0, philox.TAG_BERNOULLI)
    c2 = gb.stratified_counts(np.abs(q) / n2, np.asarray(u2, dtype=np.float64)[None])
    np.testing.assert_allclose(gb.weights(q[None], np.abs(q), c2, n2, 1)[0], n2 * qh2, rtol=1e-15)


def test_group_scores_are_unbiased():
    rng = np.random.default_rng(11)
    G, d, nk, B = 4, 16, 30, 4
    qg = rng.normal(size=(G, d))
    K = rng.normal(size=(nk, d))
    exact = (qg @ K.T) / math.sqrt(d)
    runs = np.array([gb.group_scores(qg, K, B, seed, 0, 1)[0] for seed in range(1500)])
    se = runs.std(axis=0) / math.sqrt(runs.shape[0])
    assert np.all(np.abs(runs.mean(axis=0) - exact) <= 5 * se + 1e-12)


def test_stratified_variance_falls_as_one_over_B_squared():
    """Var(mhat_i) = norm^2 Var(c_i) / B^2 with Var(c_i) = f (1 - f) <= 1/4, f the fractional part of B pi_i:
    stratification bounds the variance by norm^2 / (4 B^2) per feature (i.i.d. samples would give
    norm^2 pi (1 - pi) / B). Checked empirically: the score variance drops more than 8x from B = 1 to 8."""
    rng = np.random.default_rng(12)
    G, d, nk = 4, 32, 20
    qg = rng.normal(size=(G, d))
    K = rng.normal(size=(nk, d))
    v = {}
    for B in (1, 8):
        runs = np.array([gb.group_scores(qg, K, B, seed, 0, 0)[0] for seed in range(600)])
        v[B] = runs.var(axis=0).sum()
    assert v[8] < v[1] / 8


def test_zero_features_are_skipped_and_counts_cover_the_rest():
    qg = np.array([[0.0, 1.0, -2.0, 0.01], [0.0, -1.0, 2.0, 0.0]])
    s, c, norm = gb.group_scores(qg, np.ones((3, 4)), 4, 5, 0, 0)
    assert norm == 2.0 and c[0] == 0            # m_0 = 0: never read
    assert c[2] == 4                            # pi = 1: every sample keeps it
    assert c[1] == 2                            # B pi = 2 exactly: floor = ceil
    assert c[3] in (0, 1)                       # B pi = 0.01


def test_uniforms_are_the_published_generator():
    U = gb.uniforms(9, 2, 3, 5, 3)
    for n in range(3):
        for i in range(5):
            x = philox.philox4x32_10(i, 3, 2, gb.TAG_GROUP + 256 * n, *philox.seed_key(9))
            assert U[n, i] == philox.u53_from_words(int(x[0]), int(x[1]))


def test_decode_with_group_scores():
    rng = np.random.default_rng(2)
    q = rng.normal(size=(1, 4, 16)).astype(np.float32)
    K = rng.normal(size=(1, 300, 1, 16)).astype(np.float32)
    V = rng.normal(size=(1, 300, 1, 16)).astype(np.float32)
    s, counts = gb.scores(q, K, 4, 3)
    assert counts.shape == (1, 1, 16)
    r = oracle.decode(q, K, V, 32, oracle.STRAT, 3, out_dtype="f32", scores=s)
    p, _, _ = oracle.softmax(s[0, 2])
    np.testing.assert_allclose(r.prob[0, 2], p, rtol=1e-12)

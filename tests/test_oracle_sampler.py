"""Pins for the oracle's sampling: points, inverse CDF, estimator algebra.

References are to "Stochastic Sparse Attention for Memory-Bound Inference": Section 2 (SANTA, Eqs. 2-4),
Section 2.1 (S²ANTA strat / sys construction), Appendix A (Definition A.1, Propositions A.2-A.4,
Theorem A.6), Appendix M (variance closed forms) and Appendix O, Algorithm 5 (floor-difference
systematic counts).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import philox
from tests import enumerate_exact as ex

HERE = os.path.dirname(os.path.abspath(__file__))

# dyadic probability vectors: exact in fp64, so oracle CDFs equal the rational ones bit for bit
CASES = [
    [Fraction(k, 16) for k in (5, 1, 0, 7, 3)],
    [Fraction(k, 64) for k in (1, 2, 4, 8, 16, 33)],
    [Fraction(k, 8) for k in (1, 1, 1, 1, 1, 1, 1, 1)],
    [Fraction(k, 32) for k in (0, 31, 1)],
    [Fraction(1)],
]


def _V(nk, d=3, seed=0):
    rng = np.random.default_rng(seed)
    return rng.integers(-8, 9, size=(nk, d)).astype(np.float64)


def _fr(V):
    return [[Fraction(int(x)) for x in row] for row in V]


def test_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "worked_example.json")))
    nk, S = g["nk"], g["S"]
    V = _V(nk, d=4, seed=1)
    p = np.array([0.5, 0.25, 0.25])
    F = oracle.cdf(p)
    # points inside [0,F1), [0,F1), [F2,1): the one-hot samples key 1, key 1, key 3
    J, _ = oracle.inverse_cdf(F, p, np.array([0.1, 0.4, 0.9]))
    assert list(J + 1) == g["samples_1based"]
    est = oracle.estimate(V, J, S)
    want = (V[0] + V[0] + V[2]) / 3.0
    assert np.array_equal(est, want)
    coef = np.array(g["coefficients"])
    assert np.allclose(est, coef @ V, rtol=0, atol=1e-14)


def test_inverse_cdf_half_open_convention():
    p = np.array([0.25, 0.0, 0.5, 0.25])
    F = oracle.cdf(p)  # 0.25, 0.25, 0.75, 1.0
    T = np.array([0.0, 0.25, 0.2499999999999, 0.75, 0.7499999999, 0.999999])
    J, delta = oracle.inverse_cdf(F, p, T)
    # a point exactly on F(j) belongs to the next key; the zero-mass key 1 is never chosen
    assert list(J) == [0, 2, 0, 3, 2, 3]
    assert delta[1] == 0.0 and delta[3] == 0.0


def test_inverse_cdf_clamps_to_last_positive_key():
    p = np.array([0.5, 0.4999999999999999, 0.0])
    F = oracle.cdf(p)
    assert F[-1] < 1.0
    J, _ = oracle.inverse_cdf(F, p, np.array([1.0 - 2.0**-53]))
    assert J[0] == 1


@pytest.mark.parametrize("case", range(len(CASES)))
def test_iid_enumeration_matches_closed_forms(case):
    p = CASES[case]
    V = _V(len(p), seed=case)
    Vf = _fr(V)
    mu = [sum((p[j] * Vf[j][i] for j in range(len(p))), Fraction(0)) for i in range(V.shape[1])]
    for S in (1, 2, 3):
        if len(p) ** S > 4000:
            continue
        mean, var = ex.moments(ex.iid_joint(p, S), Vf)
        assert mean == mu  # Proposition A.2, exactly
        pf = np.array([float(x) for x in p])
        assert abs(float(var) - oracle.var_trace_iid(pf, V, S)) < 1e-12  # Proposition A.3 / Appendix M


@pytest.mark.parametrize("case", range(len(CASES)))
def test_strat_enumeration_matches_closed_forms(case):
    p = CASES[case]
    V = _V(len(p), seed=10 + case)
    Vf = _fr(V)
    mu = [sum((p[j] * Vf[j][i] for j in range(len(p))), Fraction(0)) for i in range(V.shape[1])]
    pf = np.array([float(x) for x in p])
    F = oracle.cdf(pf)
    for S in (1, 2, 3, 4):
        if len(p) ** S > 5000:
            continue
        mean, var = ex.moments(ex.strat_joint(p, S), Vf)
        assert mean == mu  # Proposition A.4 (strat), exactly
        assert abs(float(var) - oracle.var_trace_strat(F, V, S)) < 1e-12  # Appendix M closed form
        assert float(var) <= oracle.var_trace_iid(pf, V, S) + 1e-12  # Theorem A.6 / Corollary A.7


@pytest.mark.parametrize("case", range(len(CASES)))
def test_sys_enumeration_is_unbiased_and_matches_oracle(case):
    p = CASES[case]
    V = _V(len(p), seed=20 + case)
    Vf = _fr(V)
    mu = [sum((p[j] * Vf[j][i] for j in range(len(p))), Fraction(0)) for i in range(V.shape[1])]
    pf = np.array([float(x) for x in p])
    F = oracle.cdf(pf)
    for S in (1, 2, 3, 4, 8):
        pieces = list(ex.sys_pieces(p, S))
        mean, _ = ex.moments(((J, pr) for J, pr, _ in pieces), Vf)
        assert mean == mu  # Proposition A.4 (sys), exactly
        for J, _, mid in pieces:
            T = np.array([float(mid) + m / S for m in range(S)])
            got, _ = oracle.inverse_cdf(F, pf, T)
            assert tuple(got) == J


@pytest.mark.parametrize("case", range(len(CASES)))
def test_oracle_inverse_cdf_reproduces_stratum_masses(case):
    p = CASES[case]
    pf = np.array([float(x) for x in p])
    F = oracle.cdf(pf)
    N = 4096
    for S in (1, 2, 4):
        for m in range(S):
            T = (m + (np.arange(N) + 0.5) / N) / S
            J, _ = oracle.inverse_cdf(F, pf, T)
            freq = np.bincount(J, minlength=len(p)) / N
            want = np.array([float(w) for w in ex.stratum_dist(p, m, S)])
            assert np.array_equal(freq, want)


def test_sample_points_per_mode():
    S = 64
    for b, h, seed in [(0, 0, 1), (3, 17, 99), (7, 31, 2**40 + 5)]:
        Ti = oracle.sample_points(oracle.IID, S, seed, b, h)
        Ts = oracle.sample_points(oracle.STRAT, S, seed, b, h)
        Ty = oracle.sample_points(oracle.SYS, S, seed, b, h)
        m = np.arange(S)
        assert np.all((Ti >= 0) & (Ti < 1))
        assert np.all((Ts >= m / S) & (Ts < (m + 1) / S))           # one point per stratum I_m
        assert np.array_equal(Ts, (m + Ti) / S)                       # same uniforms as i.i.d.
        assert 0 <= Ty[0] < 1 / S                                     # U ~ U[0, 1/S)
        assert np.allclose(np.diff(Ty), 1 / S, rtol=0, atol=1e-15)    # T_m = U + m/S
        u = philox.uniforms(seed, 0, h, b, philox.TAG_SYS)
        assert np.array_equal(Ty, (m + u) / S)


def test_strat_and_iid_agree_at_S1():
    rng = np.random.default_rng(3)
    p = rng.dirichlet(np.ones(50))
    F = oracle.cdf(p)
    for seed in range(20):
        Ti = oracle.sample_points(oracle.IID, 1, seed, 0, 0)
        Ts = oracle.sample_points(oracle.STRAT, 1, seed, 0, 0)
        assert np.array_equal(oracle.inverse_cdf(F, p, Ti)[0], oracle.inverse_cdf(F, p, Ts)[0])


def test_strat_stratum_frequencies_statistical():
    p = CASES[0]
    pf = np.array([float(x) for x in p])
    F = oracle.cdf(pf)
    S, n = 4, 4000
    counts = np.zeros((S, len(p)))
    for seed in range(n):
        J, _ = oracle.inverse_cdf(F, pf, oracle.sample_points(oracle.STRAT, S, seed, 0, 0))
        counts[np.arange(S), J] += 1
    for m in range(S):
        want = np.array([float(w) for w in ex.stratum_dist(p, m, S)])
        sd = np.sqrt(want * (1 - want) / n)
        assert np.all(np.abs(counts[m] / n - want) <= 4 * sd + 1e-12)


def test_sys_counts_are_floor_or_ceil():
    rng = np.random.default_rng(5)
    for trial in range(30):
        nk = int(rng.integers(5, 2000))
        p = rng.dirichlet(np.full(nk, 0.3))
        F = oracle.cdf(p)
        S = int(rng.choice([7, 64, 256, 1000]))
        J, _ = oracle.inverse_cdf(F, p, oracle.sample_points(oracle.SYS, S, trial, 0, 0))
        c = np.bincount(J, minlength=nk)
        assert c.sum() == S
        assert np.all(c >= np.floor(S * p - 1e-9)) and np.all(c <= np.ceil(S * p + 1e-9))


def test_floor_difference_counts_equal_inverse_cdf_counts():
    """Appendix O, Algorithm 5 over a single tile: c_n = floor(a + S F_n) - floor(a + S F_{n-1}) with
    offset a = 1 - u is the systematic count of key n (independent formulation of S²ANTA-sys)."""
    rng = np.random.default_rng(9)
    checked = 0
    for trial in range(40):
        nk = int(rng.integers(3, 3000))
        p = rng.dirichlet(np.full(nk, 0.5))
        F = oracle.cdf(p)
        S = int(rng.choice([1, 5, 128, 512]))
        seed, b, h = trial, trial % 3, trial % 5
        u = float(philox.uniforms(seed, 0, h, b, philox.TAG_SYS))
        a = 1.0 - u
        x = a + S * np.concatenate(([0.0], F))
        c_alg5 = np.diff(np.floor(x)).astype(np.int64)
        J, _ = oracle.inverse_cdf(F, p, oracle.sample_points(oracle.SYS, S, seed, b, h))
        c_inv = np.bincount(J, minlength=nk)
        frac = np.abs(x - np.round(x))
        if np.min(frac[1:]) < 1e-9:
            continue  # a point on an interval edge: the two formulations may differ there
        assert np.array_equal(c_alg5, c_inv)
        checked += 1
    assert checked >= 30


def test_uniform_attention_systematic_reads_every_key_equally():
    nk, d, S = 64, 8, 128
    rng = np.random.default_rng(1)
    V = rng.standard_normal((1, nk, 1, d)).astype(np.float32)
    K = np.zeros((1, nk, 1, d), dtype=np.float32)  # all logits 0 -> p = 1/nk
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    r = oracle.decode(q, K, V, S, oracle.SYS, seed=4, out_dtype="f32")
    assert np.array_equal(np.bincount(r.idx[0, 0], minlength=nk), np.full(nk, 2))
    assert np.allclose(r.est[0, 0], V[0, :, 0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-15)


def test_one_hot_attention_returns_that_row():
    nk, d = 100, 16
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, d)).astype(np.float32)
    q[0, 1] = q[0, 0]
    K = rng.standard_normal((1, nk, 1, d)).astype(np.float32) * 0.01
    K[0, 37, 0] = q[0, 0] * 400.0  # logit ~ 100*|q|^2: every other key underflows to p = 0
    V = rng.standard_normal((1, nk, 1, d)).astype(np.float32)
    for mode in (oracle.IID, oracle.STRAT, oracle.SYS):
        r = oracle.decode(q, K, V, 32, mode, seed=3, out_dtype="f32")
        assert np.all(r.idx == 37)
        assert np.array_equal(r.out[0, 0], V[0, 37, 0].astype(np.float64))
        assert np.array_equal(r.out[0, 1], V[0, 37, 0].astype(np.float64))


def test_strat_and_sys_indices_are_nondecreasing():
    rng = np.random.default_rng(4)
    p = rng.dirichlet(np.full(500, 0.2))
    F = oracle.cdf(p)
    for mode in (oracle.STRAT, oracle.SYS):
        for seed in range(10):
            J, _ = oracle.inverse_cdf(F, p, oracle.sample_points(mode, 97, seed, 1, 2))
            assert np.all(np.diff(J) >= 0)


def test_iid_frequencies_match_torch_multinomial():
    """The i.i.d. sampler draws indices with the semantics of torch.multinomial(p, S, replacement=True)
    (the code on the alphasignal summary page): a two-sample chi-square test of the oracle's index counts
    against torch's over 40 960 draws from a peaked 12-key softmax, plus each against p itself."""
    import torch
    from scipy import stats

    rng = np.random.default_rng(11)
    s = rng.standard_normal(12) * 2.0
    p, _, _ = oracle.softmax(s)
    F = oracle.cdf(p)
    S, reps = 4096, 10
    counts = np.zeros(12, dtype=np.int64)
    for seed in range(reps):
        T = oracle.sample_points(oracle.IID, S, seed, 0, 0)
        J, _ = oracle.inverse_cdf(F, p, T)
        counts += np.bincount(J, minlength=12)
    gen = torch.Generator().manual_seed(1234)
    tm = torch.multinomial(torch.tensor(p), S * reps, replacement=True, generator=gen).numpy()
    tcounts = np.bincount(tm, minlength=12)
    n = S * reps
    keep = p * n >= 5  # chi-square cells with enough expected mass
    _, pv_two, _, _ = stats.chi2_contingency(np.stack([counts[keep], tcounts[keep]]))
    assert pv_two > 1e-3, pv_two
    for c in (counts, tcounts):
        assert stats.chisquare(c[keep], p[keep] / p[keep].sum() * c[keep].sum()).pvalue > 1e-3

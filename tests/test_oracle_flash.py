"""Pins of the S²ANTA-flash oracle (Section 3.3; Appendix P, Algorithms 6-8) against what the pages and
the mathematics fix: the budget rounding, a hand-worked two-tile example whose counts are forced, the
exact mean over the offsets (the merge reweighting makes the estimator unbiased for AV), the merge
weights as tile softmax masses, count conservation, and the offsets' generator."""

import math

import numpy as np
import pytest

import oracle
from oracle import flash, philox


def _softmax_av(s, V):
    p = np.exp(s - np.max(s))
    p /= p.sum()
    return p @ V, p


def test_tile_budget_rounding():
    assert flash.tile_budget(2048, 128) == 16      # the 32k operating point of Section 3.2
    assert flash.tile_budget(100, 128) == 1        # below one sample per tile: at least one
    assert flash.tile_budget(3, 2) == 2            # 1.5 rounds up
    assert flash.tile_budget(5, 2) == 3            # 2.5 rounds up
    assert flash.tile_budget(4, 3) == 1            # 1.33
    assert flash.tile_budget(5, 3) == 2            # 1.67
    assert flash.tile_budget(7, 1) == 7


def test_worked_two_tile_example_is_exact():
    """Tiles of 2 keys, s = (0, 0, ln 3, ln 3): p = (1, 1, 3, 3)/8, tile masses 1/4 and 3/4. With S = 4,
    S_tile = 2 and x_n = 2 * 1 / 2 = 1 for every key, so every count is 1 whatever a0 is, and the merge
    gives (1/4)(V0 + V1)/2 + (3/4)(V2 + V3)/2 = AV exactly."""
    s = np.array([0.0, 0.0, math.log(3.0), math.log(3.0)])
    V = np.array([[1.0, 0.0], [3.0, 2.0], [-1.0, 4.0], [5.0, -2.0]])
    want = (0.25 * (V[0] + V[1]) + 0.75 * (V[2] + V[3])) / 2.0
    av, p = _softmax_av(s, V)
    np.testing.assert_allclose(p, [0.125, 0.125, 0.375, 0.375], rtol=1e-15)
    for a0 in (0.01, 0.5, 0.99):
        e, c, _, st, W, Z = flash.head_estimate(s, V, 4, np.array([a0, 1.0 - a0]), tile=2)
        assert st == 2 and list(c) == [1, 1, 1, 1]
        np.testing.assert_allclose(W / Z, [0.25, 0.75], rtol=1e-15)
        np.testing.assert_allclose(e, want, rtol=1e-15)
        np.testing.assert_allclose(e, av, rtol=1e-14)


@pytest.mark.parametrize("seed", range(4))
def test_merge_weights_are_tile_masses(seed):
    rng = np.random.default_rng(seed)
    s = rng.normal(0, 3, 1000)
    m, u, l = oracle.prop.tile_stats(s, 64)
    W, Z = flash.merge_weights(m, l)
    _, p = _softmax_av(s, np.zeros((1000, 1)))
    mass = np.array([p[t * 64:(t + 1) * 64].sum() for t in range(m.shape[0])])
    np.testing.assert_allclose(W / Z, mass, rtol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_mean_over_offsets_is_av(seed):
    """E over a0 of each count is x_n = S_tile u_n / l_t, so E[O] = sum_t (W_t/Z) sum_n (u_n/l_t) V_n = AV
    (midpoint quadrature over a0, the same a0 in every tile: the expectation is linear per tile)."""
    rng = np.random.default_rng(40 + seed)
    nk, d = 300, 3
    s = rng.normal(0, 2, nk)
    V = rng.normal(size=(nk, d))
    av, _ = _softmax_av(s, V)
    N = 2000
    T = (nk + 63) // 64
    acc = np.zeros(d)
    for k in range(N):
        e, *_ = flash.head_estimate(s, V, 20, np.full(T, (k + 0.5) / N), tile=64)
        acc += e
    np.testing.assert_allclose(acc / N, av, atol=8.0 / N * np.abs(V).max())


@pytest.mark.parametrize("seed", range(4))
def test_counts_conserve_the_tile_budget(seed):
    rng = np.random.default_rng(60 + seed)
    nk = int(rng.integers(300, 2000))
    s = rng.normal(0, 2, nk)
    S = int(rng.integers(1, 600))
    T = (nk + 255) // 256
    a0 = rng.uniform(1e-6, 1 - 1e-6, T)
    _, c, _, st, _, _ = flash.head_estimate(s, np.zeros((nk, 1)), S, a0)
    assert st == flash.tile_budget(S, T)
    m, u, l = oracle.prop.tile_stats(s, 256)
    for t in range(T):
        ct = c[t * 256:(t + 1) * 256]
        assert ct.sum() == st
        x = st * u[t * 256:(t + 1) * 256] / l[t]
        assert np.all(np.abs(ct - x) < 1.0 + 1e-9)


def test_decode_structure_and_unbiasedness():
    rng = np.random.default_rng(5)
    B, H, Hkv, d, nk, S = 1, 2, 1, 8, 700, 30
    q = rng.normal(size=(B, H, d)).astype(np.float32)
    K = rng.normal(size=(B, nk, Hkv, d)).astype(np.float32)
    V = rng.normal(size=(B, nk, Hkv, d)).astype(np.float32)
    r = flash.decode(q, K, V, S, seed=3, out_dtype="f32")
    T = 3
    st = flash.tile_budget(S, T)
    assert r.idx.shape == (B, H, T * st) and r.extra["S_tile"] == st
    for h in range(H):
        np.testing.assert_array_equal(np.bincount(r.idx[0, h], minlength=nk), r.extra["counts"][0, h])
        for t in range(T):
            seg = r.idx[0, h, t * st:(t + 1) * st]
            assert np.all(np.diff(seg) >= 0) and seg.min() >= t * 256 and seg.max() < min(nk, (t + 1) * 256)
        np.testing.assert_allclose(flash.estimate_from_idx(V[0, :, 0], r.idx[0, h], r.extra["weights"][0, h], st),
                                   r.est[0, h], rtol=1e-12, atol=1e-12)
    # mean over seeds against the exact AV (closed form), within 5 standard errors
    Kf, Vf = K[0, :, 0].astype(np.float64), V[0, :, 0].astype(np.float64)
    av, _ = _softmax_av(oracle.scores_exact(q[0, 0], Kf), Vf)
    runs = np.array([flash.decode(q[:, :1], K, V, S, seed=k, out_dtype="f32", keep_prob=False).est[0, 0]
                     for k in range(300)])
    sd = runs.std(axis=0) / math.sqrt(runs.shape[0])
    assert np.all(np.abs(runs.mean(axis=0) - av) <= 5 * sd + 1e-12)


def test_offsets_are_the_published_generator():
    a0 = flash.offsets(9, 2, 3, 5)
    for t in range(5):
        x = philox.philox4x32_10(t, 3, 2, flash.TAG_FLASH, *philox.seed_key(9))
        assert a0[t] == philox.u53_from_words(int(x[0]), int(x[1]))

"""Pins for the oracle's score/softmax/dense path and the statistical properties of its estimators.

"Stochastic Sparse Attention for Memory-Bound Inference": Section 2, Eq. 1 (SDPA), Appendix A
(Propositions A.2-A.4: unbiasedness; Proposition A.3: variance 1/S; Theorem A.6: stratification never
increases the variance), Appendix M (variance closed forms).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads


def _tiny():
    w = workloads.make(1)
    q, K, V = w.numpy_inputs()
    return w, q, K, V


def test_scale_and_scores_match_torch():
    rng = np.random.default_rng(0)
    for d in (64, 128):
        q = rng.standard_normal(d)
        K = rng.standard_normal((300, d))
        s = oracle.scores_exact(q, K)
        ref = (torch.from_numpy(K) @ torch.from_numpy(q)).numpy() / np.sqrt(d)
        assert np.allclose(s, ref, rtol=1e-13, atol=1e-13)
    assert oracle.scale(64) == 0.125


def test_softmax_and_dense_match_torch_sdpa():
    """Eq. 1 reduces to torch's fp64 CPU scaled_dot_product_attention (GQA by repeating KV heads)."""
    q, K, V, _ = workloads.make_inputs(2, 8, 2, 64, 257, dtype="bf16", spikes_per_head=3, rng_seed=5)
    qn, Kn, Vn = q.double(), K.double(), V.double()
    mu, _ = oracle.dense(qn.numpy(), Kn.numpy(), Vn.numpy())
    G = 4
    Kt = Kn.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)  # [B, H, nk, d]
    Vt = Vn.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qn.unsqueeze(2), Kt, Vt).squeeze(2).numpy()
    assert np.allclose(mu, ref, rtol=1e-12, atol=1e-12)
    s = oracle.scores_exact(qn[1, 5].numpy(), Kn[1, :, 1].numpy())
    p, m_star, Z = oracle.softmax(s)
    assert np.allclose(p, torch.softmax(torch.from_numpy(s), dim=0).numpy(), rtol=1e-13, atol=1e-300)
    assert abs(p.sum() - 1.0) < 1e-14 and m_star == s.max()


def test_round_to_bf16_matches_torch_and_rounds_directly():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.round_to_bf16(x.astype(np.float64)), want)
    one = 1.0
    cases = {
        one + 2.0**-8: 1.0,                        # tie -> even (1.0)
        one + 3 * 2.0**-8: one + 2.0**-6,          # tie -> even (1 + 2^-6)
        one + 2.0**-8 + 2.0**-40: one + 2.0**-7,   # just above the tie: up (double rounding via fp32 would tie)
        -(one + 2.0**-8 + 2.0**-40): -(one + 2.0**-7),
        0.0: 0.0,
        2.0**-100: 2.0**-100,
    }
    for x, want in cases.items():
        assert oracle.round_to_bf16(np.array([x]))[0] == want


@pytest.mark.parametrize("mode", [oracle.IID, oracle.STRAT, oracle.SYS])
def test_unbiased_over_4096_seeds(mode):
    """E[estimate] = AV (Propositions A.2 and A.4): the mean over 4096 seeds lies within 3 sigma."""
    w, q, K, V = _tiny()
    S, n = w.S, 4096
    Kf, Vf = K[0, :, 0].astype(np.float64), V[0, :, 0].astype(np.float64)
    p, _, _ = oracle.softmax(oracle.scores_exact(q[0, 0], Kf))
    F = oracle.cdf(p)
    mu = p @ Vf
    ests = np.empty((n, Vf.shape[1]))
    for seed in range(n):
        J, _ = oracle.inverse_cdf(F, p, oracle.sample_points(mode, S, seed, 0, 0))
        ests[seed] = oracle.estimate(Vf, J, S)
    mean = ests.mean(axis=0)
    if mode == oracle.IID:
        vt = oracle.var_trace_iid(p, Vf, S)
    elif mode == oracle.STRAT:
        vt = oracle.var_trace_strat(F, Vf, S)
    else:
        vt = float(np.sum(ests.var(axis=0, ddof=1)))  # Appendix M replicate estimator for sys
    assert np.linalg.norm(mean - mu) <= 3.0 * np.sqrt(vt / n)
    # per coordinate: at most the binomial(64, 0.0027) 99.9% quantile (= 2) outside 3 sigma
    sd = ests.std(axis=0, ddof=1) / np.sqrt(n)
    assert np.sum(np.abs(mean - mu) > 3 * sd) <= 2
    if mode != oracle.SYS:
        emp = float(np.sum(ests.var(axis=0, ddof=1)))
        assert abs(emp / vt - 1.0) < 0.1  # closed form matches the empirical variance trace


def test_decode_end_to_end_equals_building_blocks():
    w, q, K, V = _tiny()
    r = oracle.decode(q, K, V, w.S, oracle.IID, seed=17, out_dtype="f32")
    Kf, Vf = K[0, :, 0].astype(np.float64), V[0, :, 0].astype(np.float64)
    p, _, _ = oracle.softmax(oracle.scores_exact(q[0, 0], Kf))
    J, _ = oracle.inverse_cdf(oracle.cdf(p), p, oracle.sample_points(oracle.IID, w.S, 17, 0, 0))
    assert np.array_equal(r.idx[0, 0], J)
    assert np.array_equal(r.est[0, 0], oracle.estimate(Vf, J, w.S))
    assert np.array_equal(r.out[0, 0], r.est[0, 0].astype(np.float32).astype(np.float64))
    assert np.allclose(r.mu[0, 0], p @ Vf)


def test_variance_scales_as_one_over_S_and_strat_dominates():
    """Proposition A.3 (IID variance = tr(Sigma)/S) and Theorem A.6 (strat <= iid)."""
    rng = np.random.default_rng(3)
    for _ in range(5):
        nk, d = 400, 16
        p = rng.dirichlet(np.full(nk, 0.1))
        V = rng.standard_normal((nk, d))
        F = oracle.cdf(p)
        base = oracle.var_trace_iid(p, V, 1)
        for S in (1, 4, 16, 64):
            assert np.isclose(oracle.var_trace_iid(p, V, S) * S, base, rtol=1e-12)
            assert oracle.var_trace_strat(F, V, S) <= oracle.var_trace_iid(p, V, S) * (1 + 1e-12)


def test_unique_rows_and_bytes():
    q, K, V, _ = workloads.make_inputs(1, 8, 2, 64, 512, dtype="bf16", spikes_per_head=4, rng_seed=8)
    r = oracle.decode(q.float().numpy(), K.float().numpy(), V.float().numpy(), 32, oracle.STRAT, seed=2)
    for kv in range(2):
        union = np.unique(r.idx[0, kv * 4:(kv + 1) * 4])
        assert r.unique[0, kv] == union.size <= min(512, 4 * 32)  # U <= min(nk, G*S)
    bt = oracle.bytes_touched(1, 512, 8, 2, 64, 2, int(r.unique.sum()))
    assert bt["bytes_k"] == 512 * 2 * 64 * 2
    assert bt["bytes_v"] == int(r.unique.sum()) * 64 * 2
    assert bt["bytes_total"] == bt["bytes_k"] + bt["bytes_v"] + 2 * 8 * 64 * 2

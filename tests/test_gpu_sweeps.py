"""Variance and unique-key measurements through the GPU kernels ("Stochastic Sparse Attention for
Memory-Bound Inference", Appendix L and Appendix M protocol), checked against the oracle's closed forms:
the replicate variance trace of the GPU's SANTA and S²ANTA-strat estimates over independent seeds must
match tr(Sigma)/S and (1/S^2) sum_m tr(Sigma_m); SANTA, the stratified and systematic variants and
S²ANTA-flash must be unbiased (mean squared error against the exact AV equals the variance trace), while
S²ANTA-prop's deterministic largest-remainder budgets leave the bias of its closed-form expectation
sum_t (S_t/S) sum_n (u_n/l_t) V_n; unique keys are bounded by S and nk and grow with S."""

import numpy as np
import pytest
import torch

import oracle
import stochastic_sparse_attention_split_amd as santa
import workloads
from tests.parity import log

pytestmark = pytest.mark.gpu

B, H, HKV, D, NK = 1, 4, 1, 64, 2048
R = 400


@pytest.fixture(scope="module")
def inputs():
    q, K, V, _ = workloads.make_inputs(B, H, HKV, D, NK, dtype="f32", spikes_per_head=8, rng_seed=4242)
    qn, Kn, Vn = q.numpy().astype(np.float64), K.numpy().astype(np.float64), V.numpy().astype(np.float64)
    ps, Fs, mus, ss = [], [], [], []
    for h in range(H):
        s = oracle.scores_exact(qn[0, h], Kn[0, :, 0])
        p, _, _ = oracle.softmax(s)
        ss.append(s)
        ps.append(p)
        Fs.append(oracle.cdf(p))
        mus.append(p @ Vn[0, :, 0])
    dev = torch.device("cuda:0")
    return q.to(dev), K.to(dev), V.to(dev), Vn[0, :, 0], ps, Fs, np.array(mus), ss


def _replicates(q, K, V, S, mode):
    dev = q.device
    L = santa.samples_per_head(NK, S, mode)
    ws = santa.new_workspace(santa.workspace_bytes(B, NK, H, HKV, D, S, mode), dev)
    idx = torch.empty((B, H, L), dtype=torch.int32, device=dev)
    est = np.zeros((R, H, D))
    uniq = np.zeros((R, H))
    for r in range(R):
        o = santa.decode(q, K, V, S, mode, 1000 + r, workspace=ws, idx_out=idx)
        est[r] = o.double().cpu().numpy()[0]
        ih = idx.cpu().numpy()[0]
        uniq[r] = [np.unique(ih[h]).size for h in range(H)]
    return est, uniq


@pytest.mark.parametrize("S", [16, 128])
@pytest.mark.parametrize("mode", ["iid", "strat", "sys", "prop", "flash"])
def test_variance_trace_and_unbiasedness(inputs, mode, S):
    q, K, V, Vn, ps, Fs, mus, ss = inputs
    log(f"sweep {mode} S={S}")
    est, uniq = _replicates(q, K, V, S, mode)
    vt = ((est - est.mean(axis=0)) ** 2).sum(axis=2).sum(axis=0) / (R - 1)      # per head
    mse = ((est - mus[None]) ** 2).sum(axis=2).mean(axis=0)                      # per head
    if mode == "prop":
        expect = np.array([oracle.prop.expected_estimate(ss[h], Vn, S) for h in range(H)])
    else:
        expect = mus
    bias2 = ((expect - mus) ** 2).sum()
    log(f"  vartrace {vt.sum():.5g}  mse {mse.sum():.5g}  bias^2 {bias2:.3g}  U {uniq.mean():.2f}")
    # the squared error against the exact AV is the variance plus the squared bias of the expectation
    assert abs(mse.sum() / (vt.sum() + bias2) - 1.0) < 0.2
    # and the replicates' mean is that expectation, within 5 standard errors per coordinate
    se = est.std(axis=0) / np.sqrt(R)
    assert np.all(np.abs(est.mean(axis=0) - expect) <= 5 * se + 1e-9)
    if mode == "iid":
        want = sum(oracle.var_trace_iid(ps[h], Vn, S) for h in range(H))
        log(f"  closed form {want:.5g}")
        assert abs(vt.sum() / want - 1.0) < 0.15
    if mode == "strat":
        want = sum(oracle.var_trace_strat(Fs[h], Vn, S) for h in range(H))
        log(f"  closed form {want:.5g}")
        assert abs(vt.sum() / want - 1.0) < 0.15
    L = santa.samples_per_head(NK, S, mode)
    assert np.all(uniq >= 1) and np.all(uniq <= min(NK, L))


def test_unique_keys_grow_with_S(inputs):
    q, K, V, *_ = inputs
    for mode in ("iid", "strat", "sys"):
        means = []
        for S in (8, 32, 128):
            _, uniq = _replicates(q, K, V, S, mode)
            means.append(uniq.mean())
        log(f"unique keys {mode}: {means}")
        assert means[0] < means[1] < means[2]

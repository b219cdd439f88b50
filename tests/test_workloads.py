"""The seeded input generator: shapes, determinism and the planted structure it promises."""

import numpy as np
import torch

import workloads


def test_shapes_dtypes_and_determinism():
    a = workloads.make(2, nk=2048)
    b = workloads.make(2, nk=2048)
    assert a.q.shape == (1, 32, 128) and a.K.shape == (1, 2048, 8, 128) and a.V.shape == a.K.shape
    assert a.K.dtype == torch.bfloat16
    assert torch.equal(a.K, b.K) and torch.equal(a.q, b.q) and torch.equal(a.V, b.V)
    t = workloads.make(1)
    assert t.K.dtype == torch.float32 and t.K.shape == (1, 1024, 1, 64)


def test_planted_spikes_are_aligned_and_distinct_within_group():
    q, K, V, _ = workloads.make_inputs(1, 8, 2, 128, 4096, dtype="bf16", spikes_per_head=16, rng_seed=3)
    qf, Kf = q.double().numpy(), K.double().numpy()
    for kv in range(2):
        hits = []
        for g in range(4):
            h = kv * 4 + g
            cos = (Kf[0, :, kv] @ qf[0, h]) / (np.linalg.norm(Kf[0, :, kv], axis=1) * np.linalg.norm(qf[0, h]))
            top = np.nonzero(cos > 0.8)[0]
            assert len(top) == 16
            assert np.all(np.abs(cos[top] - 0.9) < 0.01)
            hits.append(top)
        assert len(np.unique(np.concatenate(hits))) == 64


def test_recency_bump_raises_group_logits():
    nk, d = 2048, 128
    q, K0, _, _ = workloads.make_inputs(1, 7, 1, d, nk, dtype="f32", recency=0, rng_seed=11)
    q, K1, _, _ = workloads.make_inputs(1, 7, 1, d, nk, dtype="f32", recency=512, rng_seed=11)
    qf = q.double().numpy()[0]
    s0 = K0.double().numpy()[0, :, 0] @ qf.T / np.sqrt(d)
    s1 = K1.double().numpy()[0, :, 0] @ qf.T / np.sqrt(d)
    rise = s1 - s0
    assert np.all(rise[-512:] >= 2.0 - 1e-4)
    assert np.allclose(rise[:-512], 0.0)

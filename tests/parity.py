"""Shared comparison of one GPU decode against the oracle (used by the GPU parity tests and smoke()).

Tolerances (fixed for this operator):
  * probabilities: |p_gpu - p_oracle| <= 1e-3 * p_oracle (+1e-300 for underflowed keys);
  * indices: equal, except where the oracle's point lies within 1e-6 of an edge of its CDF interval;
    such excused mismatches must number at most 1e-4 of the samples;
  * outputs: max-abs 2e-2 for bf16 and 1e-5 for fp32; a head with an excused mismatch is compared
    against the oracle's gather of the GPU's own indices instead.
"""

from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import stochastic_sparse_attention_split_amd as santa

P_RTOL = 1e-3
EDGE = 1e-6
EDGE_PROP = 1e-9   # S²ANTA-prop: distance of a0 + p to an integer at which a count may flip
MISMATCH_FRAC = 1e-4
OUT_ATOL = {"bf16": 2e-2, "f32": 1e-5}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(q, K, V, S, mode, seed, ternary, dtype, want_prob=True, nk=None, kfm=False, group_b=0):
    dev = torch.device("cuda:0")
    qd, Kd, Vd = q.to(dev), K.to(dev), V.to(dev)
    if kfm:
        Kd = santa.feature_major(Kd)
    B, H, d = q.shape
    n_keys = K.shape[1] if nk is None else nk
    idx = torch.empty((B, H, santa.samples_per_head(n_keys, S, mode)), dtype=torch.int32, device=dev)
    prob = torch.empty((B, H, n_keys), dtype=torch.float64, device=dev) if want_prob else None
    out, info = santa.decode(qd, Kd, Vd, S, mode, seed, ternary=ternary, nk=nk, idx_out=idx, prob_out=prob,
                             stats=True, k_feature_major=kfm, group_bernoulli=group_b)
    torch.cuda.synchronize()
    return out, idx, prob, info


def _feature_rows(qn, Kn, seed, ternary, group_b, group_counts):
    """Feature rows of K^T the feature-major score pass reads: features with a non-zero weight for some
    head of the group (mean-group Bernoulli: c_i > 0; ternary: qhat != 0 for some head; exact: q != 0)."""
    B, H, d = qn.shape
    Hkv = Kn.shape[2]
    G = H // Hkv
    rows = 0
    for b in range(B):
        for kv in range(Hkv):
            if group_b:
                rows += int((group_counts[b, kv] > 0).sum())
            elif ternary:
                hit = np.zeros(d, dtype=bool)
                for g in range(G):
                    hit |= oracle.ternary_query(qn[b, kv * G + g], seed, b, kv * G + g)[0] != 0.0
                rows += int(hit.sum())
            else:
                rows += int((np.abs(qn[b, kv * G:(kv + 1) * G]).sum(axis=0) > 0).sum())
    return rows


def compare(q, K, V, S, mode: str, seed: int, *, ternary=False, dtype="bf16", want_prob=True, ref=None,
            nk=None, label="", kfm=False, group_b=0):
    """Run GPU and oracle on the same inputs; assert the parity contract; return a report dict.
    kfm: K is handed to the library feature-major; group_b > 0: mean-group-query Bernoulli scores."""
    t0 = time.time()
    out, idx, prob, info = run_gpu(q, K, V, S, mode, seed, ternary, dtype, want_prob, nk, kfm, group_b)
    if nk is not None:
        K, V = K[:, :nk], V[:, :nk]
    qn, Kn, Vn = q.float().numpy(), K.float().numpy(), V.float().numpy()
    t1 = time.time()
    sc, gcounts = (oracle.group_bernoulli.scores(qn, Kn, group_b, seed) if group_b else (None, None))
    if ref is not None:
        r = ref
    elif mode == "prop":
        r = oracle.prop.decode(qn, Kn, Vn, S, seed, out_dtype=dtype, ternary=ternary, keep_prob=want_prob,
                               scores=sc)
    elif mode == "flash":
        r = oracle.flash.decode(qn, Kn, Vn, S, seed, out_dtype=dtype, ternary=ternary, keep_prob=want_prob,
                                scores=sc)
    else:
        r = oracle.decode(qn, Kn, Vn, S, oracle.MODES[mode], seed, out_dtype=dtype, ternary=ternary,
                          keep_prob=want_prob, scores=sc)
    edge = EDGE_PROP if mode in ("prop", "flash") else EDGE
    t2 = time.time()
    rep = {"label": label, "gpu_s": t1 - t0, "oracle_s": t2 - t1}

    if want_prob:
        pg = prob.cpu().numpy()
        po = r.prob
        err = np.abs(pg - po)
        bad = err > P_RTOL * po + 1e-300
        rep["prob_max_rel"] = float(np.max(err / np.maximum(po, 1e-300)))
        assert not np.any(bad), f"{label}: {int(bad.sum())} probabilities off by more than 1e-3 relative"

    ig = idx.cpu().numpy().astype(np.int64)
    mism = ig != r.idx
    nmis = int(mism.sum())
    rep["samples"] = int(ig.size)
    rep["mismatches"] = nmis
    rep["near_edge"] = int((r.delta < edge).sum())
    if nmis:
        assert np.all(r.delta[mism] < edge), f"{label}: index mismatch away from a CDF edge"
        assert nmis <= MISMATCH_FRAC * ig.size, f"{label}: {nmis} excused mismatches > 1e-4 of {ig.size}"
    assert ig.min() >= 0 and ig.max() < Kn.shape[1]

    og = to_np_f64(out)
    B, H, d = og.shape
    G = H // Kn.shape[2]
    tol = OUT_ATOL[dtype]
    rnd = oracle.round_to_bf16 if dtype == "bf16" else oracle.round_to_f32
    worst = 0.0
    exact = 0
    for b in range(B):
        for h in range(H):
            if mism[b, h].any() and mode == "flash":
                want = rnd(oracle.flash.estimate_from_idx(np.asarray(Vn[b, :, h // G], dtype=np.float64), ig[b, h],
                                                          r.extra["weights"][b, h], r.extra["S_tile"]))
            elif mism[b, h].any():
                want = rnd(oracle.estimate(np.asarray(Vn[b, :, h // G], dtype=np.float64), ig[b, h], S))
            else:
                want = r.out[b, h]
            e = float(np.max(np.abs(og[b, h] - want)))
            worst = max(worst, e)
            exact += int(np.array_equal(og[b, h], want))
    rep["out_max_abs"] = worst
    rep["heads_bit_exact"] = exact
    rep["heads"] = B * H
    assert worst <= tol, f"{label}: output max-abs {worst} > {tol}"

    # accounting
    Ug = None
    if not nmis:
        Ug = int(info["unique_rows"])
        assert Ug == int(r.unique.sum()), f"{label}: unique rows {Ug} != oracle {int(r.unique.sum())}"
        assert info["group_unique_rows"] == [int(x) for x in np.asarray(r.unique).reshape(-1)], \
            f"{label}: distinct rows per (sequence, KV head) differ from the oracle's"
    assert sum(info["group_unique_rows"]) == info["unique_rows"]
    esz = 2 if dtype == "bf16" else 4
    if kfm:
        rows = _feature_rows(qn, Kn, seed, ternary, group_b, gcounts)
        rep["k_feature_fraction"] = rows / (B * Kn.shape[2] * d)
        assert info["bytes_k"] == rows * Kn.shape[1] * esz, f"{label}: K bytes {info['bytes_k']} != {rows} rows"
    else:
        assert info["bytes_k"] == B * Kn.shape[1] * Kn.shape[2] * d * esz
    if mode == "flash" and info["launches"] == 2:
        # fused S²ANTA-flash: each head reads its own distinct sampled rows of each tile (the GPU's samples)
        St = int(r.extra["S_tile"])
        tiles = np.sort(ig.reshape(B, H, -1, St), axis=-1)
        read = int(tiles.shape[0] * tiles.shape[1] * tiles.shape[2] + (np.diff(tiles, axis=-1) != 0).sum())
        assert read >= info["unique_rows"]
        assert info["bytes_v"] == read * d * esz, f"{label}: V bytes {info['bytes_v']} != {read} rows read"
        rep["rows_read"] = read
    else:
        assert info["bytes_v"] == info["unique_rows"] * d * esz
    assert info["launches"] >= 1
    rep["unique_rows"] = int(info["unique_rows"])
    return rep, r, out, idx

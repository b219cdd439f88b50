"""Benchmark of one S²ANTA decode layer-step on one MI355X.

Workload (default): Llama-3.1-8B-shaped single-layer decode, batch 1, 32 query / 8 KV heads, d=128,
bf16 K/V cache of nk=32768 positions with 32 planted aligned keys per query head, stratified sampling
with S=256 (seeded synthetic inputs, resident in HBM before timing).

A step is one call of santa_decode_ex, timed with HIP events on the launching stream. On this workload
the call is one kernel launch (score phase, exchange of the chunk statistics, chunk CDF, sampling,
gather, output sum), as it is for S2ANTA-prop and -flash on it; other shapes run score -> sampling+gather
per chunk -> merge. Before every timed step a 1 GiB in-place
update evicts K/V from the caches (the 256 MB Infinity Cache would otherwise hold the 64 MiB K), outside
the events, like the cold-cache protocol of the paper's kernel benchmark (Appendix Q). Reported alongside:
  * the dense bf16 decode baseline of the same library on the same inputs and protocol;
  * the roofline of the dominant kernel (the one-launch decode kernel where it runs, else the score
    kernel): its algorithmic bytes over its time from HIP events recorded with its launch (its dispatch
    and execution; a separate pass, same protocol); its measured HBM bytes from the committed rocprofv3
    counter record while the kernel sources are unchanged; the device's read rate on the same K bytes from
    a streaming-read probe timed the same way;
  * the same step captured into a HIP graph and replayed (same protocol);
  * S2ANTA-prop, S2ANTA-flash, feature-major K^T variants and one GPU's share of an 8-way head split;
  * the fp64 oracle timed on the host's cores on the same inputs (a baseline, not the target).

Prints one JSON line. --gpus N > 1 is refused: the benchmark runs on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "decode attention µs/layer-step + achieved HBM GB/s, 32k ctx, 32q/8kv d128 S=256"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--S", type=int, default=None, help="sample count override (the workload's own S by default)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-prop", action="store_true", help="skip the S2ANTA-prop (S=128), S2ANTA-flash "
                                                           "(S=2048), feature-major and head-parallel share "
                                                           "measurements")
    ap.add_argument("--profile-steps", action="store_true", help="minimal run for profilers: no CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 5 plain 64 MiB device copies (scale reference for hardware byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark: unique keys and variance trace vs S for every sampling mode "
                         "(Appendix L/M protocol) on a planted-spike 8k-token single-query input; one JSON line")
    ap.add_argument("--replicates", type=int, default=256, help="independent seeds per (mode, S) in --sweep")
    return ap.parse_args()


def source_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


KERNEL_SOURCES = ("stochastic_sparse_attention_split_amd/csrc/stream_kernel.h",
                  "stochastic_sparse_attention_split_amd/csrc/fused.hip",
                  "stochastic_sparse_attention_split_amd/csrc/common.h")


def sources_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_record():
    """Measured HBM bytes per launch of the one-launch decode kernel from committed rocprofv3 counter runs,
    if its sources are unchanged since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "decode_kernel_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("sources_sha256_16") != sources_hash():
        return None
    return rec.get("bytes_per_launch")


SWEEP_S = (32, 64, 128, 256, 512, 1024)
SWEEP_MODES = ("iid", "strat", "sys", "prop", "flash")


def run_sweep(args, santa, workloads, torch, np, dev):
    """Unique keys and variance trace vs S ("Stochastic Sparse Attention for Memory-Bound Inference",
    Appendix L, Table 17, and Appendix M): per head, U = number of distinct sampled keys and the
    replicate estimate VarTrace = (1/(R-1)) sum_r ||est_r - mean_r est||^2 over R independent seeds, plus
    the mean squared error against the dense softmax(qK^T/sqrt(d))V of the same library. fp32 inputs and
    outputs (bf16 output rounding would blur the variance at large S); the heads' values are averaged."""
    B, H, Hkv, d, nk = 1, 8, 2, 128, 8192
    q, K, V, info = workloads.make_inputs(B, H, Hkv, d, nk, dtype="f32", spikes_per_head=32, rng_seed=1017)
    q, K, V = q.to(dev), K.to(dev), V.to(dev)
    mu = santa.dense_decode(q, K, V).double()
    R = max(2, args.replicates)
    rows = []
    for mode in SWEEP_MODES:
        for S in SWEEP_S:
            L = santa.samples_per_head(nk, S, mode)
            ws = santa.new_workspace(santa.workspace_bytes(B, nk, H, Hkv, d, S, mode), dev)
            idx = torch.empty((B, H, L), dtype=torch.int32, device=dev)
            est = torch.empty((R, B, H, d), dtype=torch.float64, device=dev)
            uniq = np.zeros((R, H))
            for r in range(R):
                o = santa.decode(q, K, V, S, mode, r, workspace=ws, idx_out=idx)
                est[r] = o.double()
                ih = idx.cpu().numpy()[0]
                uniq[r] = [np.unique(ih[h]).size for h in range(H)]
            m = est.mean(dim=0, keepdim=True)
            vt = ((est - m) ** 2).sum(dim=3).sum(dim=0) / (R - 1)          # [B, H]
            mse = ((est - mu.unsqueeze(0)) ** 2).sum(dim=3).mean(dim=0)     # [B, H]
            rows.append({"mode": mode, "S": S, "samples_per_head": L, "U": round(float(uniq.mean()), 2),
                         "vartrace": float(vt.mean()), "mse_vs_dense": float(mse.mean())})
    return {"sweep": "unique keys and variance trace vs S (Appendix L/M protocol)",
            "workload": f"B{B} H{H}/Hkv{Hkv} d{d} nk{nk} f32, 32 planted keys/head, input seed 1017",
            "replicates": R, "rows": rows}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); a multi-GPU sharding of this "
              "operator is not built.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import stochastic_sparse_attention_split_amd as santa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    santa.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.sweep:
        print(json.dumps(run_sweep(args, santa, workloads, torch, np, dev)), flush=True)
        return

    w = workloads.make(args.config, S=args.S)
    q, K, V = w.q.to(dev), w.K.to(dev), w.V.to(dev)
    ternary = w.ternary
    out = torch.empty_like(q)
    ws = santa.new_workspace(santa.workspace_bytes(w.B, w.nk, w.H, w.Hkv, w.d, w.S), dev)
    dws = torch.empty(santa.dense_workspace_bytes(w.B, w.nk, w.H, w.Hkv, w.d), dtype=torch.uint8, device=dev)
    dout = torch.empty_like(q)
    thrash = torch.zeros((1 << 30) // 4, dtype=torch.float32, device=dev)

    def step():
        santa.decode(q, K, V, w.S, w.mode, w.seed, ternary=ternary, out=out, workspace=ws, stream=stream)

    def dense_step():
        santa.dense_decode(q, K, V, out=dout, workspace=dws, stream=stream)

    def timed(fn, n, cold=True):
        times = []
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            if cold:
                thrash.add_(1.0)
            starts[i].record(stream)
            fn()
            ends[i].record(stream)
        torch.cuda.synchronize()
        for i in range(n):
            times.append(starts[i].elapsed_time(ends[i]) * 1e3)  # us
        return times

    # stats of one call (launches, unique rows, bytes)
    _, info = santa.decode(q, K, V, w.S, w.mode, w.seed, ternary=ternary, out=out, workspace=ws, stats=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    us = timed(step, args.steps, cold=True)
    us_warm = timed(step, args.steps, cold=False)

    # the same step captured once into a HIP graph and replayed (the library allocates, synchronises and
    # clears nothing on this path, so the capture holds exactly its kernel launches)
    us_graph, graph_error = None, None
    try:  # an optional measurement: a capture failure is reported, not fatal to the benchmark line
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            santa.decode(q, K, V, w.S, w.mode, w.seed, ternary=ternary, out=out, workspace=ws)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            santa.decode(q, K, V, w.S, w.mode, w.seed, ternary=ternary, out=out, workspace=ws)
        for _ in range(args.warmup):
            graph.replay()
        us_graph = timed(graph.replay, args.steps, cold=True)
        del graph
    except RuntimeError as exc:
        graph_error = str(exc)[:200]
        torch.cuda.synchronize()

    # per-kernel times from events between the launches (separate pass, same protocol)
    stage = []
    for _ in range(args.steps):
        thrash.add_(1.0)
        _, si = santa.decode(q, K, V, w.S, w.mode, w.seed, ternary=ternary, out=out, workspace=ws, stage_ms=True)
        stage.append(si["stage_ms"])
    stage = np.array(stage) * 1e3  # us
    score_us = float(np.mean(stage[:, 0]))

    prop_us = None
    if not args.no_prop:  # S²ANTA-prop at the paper's 32k operating point (S = 128), same protocol
        def prop_step():
            santa.decode(q, K, V, 128, "prop", w.seed, ternary=ternary, out=out, workspace=ws, stream=stream)

        for _ in range(args.warmup):
            prop_step()
        prop_us = timed(prop_step, args.steps, cold=True)

    flash_us = None
    if not args.no_prop:  # S²ANTA-flash at its 32k operating point (S = 2048), same protocol
        ws_f = santa.new_workspace(santa.workspace_bytes(w.B, w.nk, w.H, w.Hkv, w.d, 2048, "flash"), dev)

        def flash_step():
            santa.decode(q, K, V, 2048, "flash", w.seed, ternary=ternary, out=out, workspace=ws_f, stream=stream)

        for _ in range(args.warmup):
            flash_step()
        flash_us = timed(flash_step, args.steps, cold=True)

    fm = {}
    if not args.no_prop:  # feature-major K^T: exact scores and the mean-group-query Bernoulli scores
        Kt = santa.feature_major(K)
        info_fm = {}

        def fm_step(gb):
            return santa.decode(q, Kt, V, w.S, w.mode, w.seed, out=out, workspace=ws, stream=stream,
                                k_feature_major=True, group_bernoulli=gb)

        for gb in (0, 4, 8):
            for _ in range(args.warmup):
                fm_step(gb)
            us_fm = timed(lambda: fm_step(gb), args.steps, cold=True)
            _, inf = santa.decode(q, Kt, V, w.S, w.mode, w.seed, out=out, workspace=ws, stats=True,
                                  k_feature_major=True, group_bernoulli=gb)
            key = "feature_major_exact" if gb == 0 else f"feature_major_group_bernoulli_B{gb}"
            fm[key] = {"us_median": round(statistics.median(us_fm), 3),
                       "k_rows_read_fraction": round(inf["bytes_k"] / info["bytes_k"], 4)}
        del Kt

    tp = None
    if not args.no_prop and w.Hkv % 8 == 0:  # one GPU's share of an 8-way head-parallel split, own cache
        hk, G = w.Hkv // 8, w.H // w.Hkv
        q8 = q[:, :hk * G].contiguous()
        K8, V8 = K[:, :, :hk].contiguous(), V[:, :, :hk].contiguous()
        out8, dout8 = torch.empty_like(q8), torch.empty_like(q8)
        ws8 = santa.new_workspace(santa.workspace_bytes(w.B, w.nk, hk * G, hk, w.d, w.S), dev)
        dws8 = torch.empty(santa.dense_workspace_bytes(w.B, w.nk, hk * G, hk, w.d), dtype=torch.uint8, device=dev)

        def tp_step():
            santa.decode(q8, K8, V8, w.S, w.mode, w.seed, ternary=ternary, out=out8, workspace=ws8, stream=stream)

        def tp_dense():
            santa.dense_decode(q8, K8, V8, out=dout8, workspace=dws8, stream=stream)

        for _ in range(args.warmup):
            tp_step()
            tp_dense()
        tp_us = timed(tp_step, args.steps, cold=True)
        tpd_us = timed(tp_dense, args.steps, cold=True)
        _, inf8 = santa.decode(q8, K8, V8, w.S, w.mode, w.seed, ternary=ternary, out=out8, workspace=ws8,
                               stats=True)
        tp = {"heads": hk * G, "kv_heads": hk, "us_median": round(statistics.median(tp_us), 3),
              "launches": int(inf8["launches"]), "bytes_k": int(inf8["bytes_k"]),
              "dense_bf16_us_median": round(statistics.median(tpd_us), 3)}
        tp["speedup_vs_dense"] = round(tp["dense_bf16_us_median"] / tp["us_median"], 3)
        del q8, K8, V8, ws8, dws8

    # the device's streaming read rate on the same K bytes under the same cold protocol, timed like the
    # decode kernel (events recorded with the launch: its dispatch and execution): the practical ceiling
    # of the K stream, beside the published peak
    rscratch = torch.empty(int(santa.lib().santa_stream_read_scratch_bytes()), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        santa.stream_read(K, rscratch, stream)
    read_us = []
    for _ in range(args.steps):
        thrash.add_(1.0)
        read_us.append(santa.stream_read(K, rscratch, stream, kernel_time=True)[1] * 1e3)
    read_GBps = K.numel() * K.element_size() / (statistics.median(read_us) * 1e-6) / 1e9

    dense_us = None
    if not args.no_dense:
        for _ in range(args.warmup):
            dense_step()
        dense_us = timed(dense_step, args.steps, cold=True)

    med = statistics.median(us)
    mean = statistics.fmean(us)
    esz = 2 if w.dtype == "bf16" else 4
    alg_bytes = info["bytes_k"] + info["bytes_v"] + info["bytes_qo"]
    one_launch = int(info["launches"]) == 1
    if one_launch:  # the one kernel is the whole step: its algorithmic bytes are the step's
        kernel_name = "one-launch decode (score, chunk CDF, sampling, gather, output sum)"
        kernel_bytes = alg_bytes
        traffic = traffic_record()
    else:
        kernel_name = "score (split-K fp64 MFMA scores + chunk max/sum-exp + in-chunk prefix)"
        kernel_bytes = info["bytes_k"] + w.B * w.H * w.d * esz
        traffic = None
    achieved = kernel_bytes / (score_us * 1e-6) / 1e9

    res = {
        "metric": METRIC,
        "value": round(med, 3),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "input_dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: B{w.B} H{w.H}/Hkv{w.Hkv} d{w.d} nk{w.nk} {w.dtype} {w.mode} S{w.S}"
                        f"{' ternary-q' if ternary else ''}, {w.info.get('spikes_per_head', 0)} planted keys/head",
            "batch": w.B, "heads": w.H, "kv_heads": w.Hkv, "d": w.d, "nk": w.nk, "S": w.S, "mode": w.mode,
            "seed": w.seed, "cache": "cold (1 GiB thrash before each step)",
        },
        "hbm_GBps": round(alg_bytes / (med * 1e-6) / 1e9, 1),
        "hbm_frac_of_peak": round(alg_bytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "bytes_touched": int(alg_bytes),
        "bytes": {"k": int(info["bytes_k"]), "v": int(info["bytes_v"]), "q_out": int(info["bytes_qo"])},
        "unique_rows": int(info["unique_rows"]),
        "launches": int(info["launches"]),
        "us_median": round(med, 3),
        "us_mean": round(mean, 3),
        "us_min": round(min(us), 3),
        "us_warm_median": round(statistics.median(us_warm), 3),
        "us_graph_replay_median": round(statistics.median(us_graph), 3) if us_graph else None,
        "stage_us_mean": ({"decode_kernel": round(score_us, 3),
                           "total_with_events": round(float(np.mean(stage[:, 3])), 3)} if one_launch else
                          {"score": round(score_us, 3), "cdf_resolve": round(float(np.mean(stage[:, 1])), 3),
                           "merge": round(float(np.mean(stage[:, 2])), 3),
                           "total_with_events": round(float(np.mean(stage[:, 3])), 3)}),
        "roofline": {
            "kernel": kernel_name,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "traffic_over_algorithmic": round(traffic / kernel_bytes, 4) if traffic else None,
            "kernel_us_mean": round(score_us, 3),
            "algorithmic_bytes": int(kernel_bytes),
            "measured_read_peak": round(read_GBps, 1),
            "frac_of_measured_read_peak": round(achieved / read_GBps, 4),
        },
        "stream_read_K": {"bytes": int(K.numel() * K.element_size()), "kernel_us_median": round(statistics.median(read_us), 3),
                          "GBps": round(read_GBps, 1)},
    }
    if dense_us is not None:
        dmed = statistics.median(dense_us)
        res["dense_bf16_us_median"] = round(dmed, 3)
        res["speedup_vs_dense"] = round(dmed / med, 3)
    if prop_us is not None:
        pmed = statistics.median(prop_us)
        res["s2anta_prop_S128"] = {"us_median": round(pmed, 3), "us_mean": round(statistics.fmean(prop_us), 3)}
        if dense_us is not None:
            res["s2anta_prop_S128"]["speedup_vs_dense"] = round(statistics.median(dense_us) / pmed, 3)
    for k_, v_ in fm.items():
        res[k_] = v_
    if flash_us is not None:
        fmed = statistics.median(flash_us)
        res["s2anta_flash_S2048"] = {"us_median": round(fmed, 3), "us_mean": round(statistics.fmean(flash_us), 3)}
        if dense_us is not None:
            res["s2anta_flash_S2048"]["speedup_vs_dense"] = round(statistics.median(dense_us) / fmed, 3)

    if tp is not None:
        res["head_parallel_share_of_8"] = tp

    if graph_error:
        res["graph_replay_error"] = graph_error
    if args.copy_calibration:
        src = torch.ones((64 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            thrash.add_(1.0)
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = {"read": 64 << 20, "write": 64 << 20, "copies": 5}

    if not args.no_cpu_baseline and not args.profile_steps:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle on the host's cores, same inputs, whole layer-steps until the time budget is spent."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    qn, Kn, Vn = w.numpy_inputs()
    times = []
    t_end = time.time() + budget_s
    while time.time() < t_end or not times:
        t0 = time.perf_counter()
        oracle.decode(qn, Kn, Vn, w.S, oracle.MODES[w.mode], w.seed, out_dtype=w.dtype, ternary=w.ternary,
                      keep_prob=False)
        times.append(time.perf_counter() - t0)
    return {
        "value": round(float(np.median(times)) * 1e6, 1),
        "unit": "us/layer-step",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(times)} whole layer-steps of the benchmark workload (all {w.H} heads, nk={w.nk}), "
                  f"median; host has {os.cpu_count()} CPUs, {len(os.sched_getaffinity(0))} in affinity",
    }


if __name__ == "__main__":
    main()

"""Benchmark: latent MLA decode on one MI355X, batch 16 at kv ~68,430, fp8.

One step = one mla_decode call (plan, index fetch, row gather, QK^T, online
softmax, P.V, split epilogue and combine) over one layer's inputs.  Like a
model step, consecutive steps cycle through `--layers` independent layer
caches (same requests and index lists, separate pools and queries), so a
layer's distinct rows are evicted from the last-level cache before the same
layer comes round again.  Inputs are resident in HBM before timing starts.

Prints one JSON line.  `value` is algorithmic GB/s: per call,
sum(kv_len) * (576 + 4) + |q| + |o| bytes (the issue's own accounting) over
the measured time per call.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode µs/call + HBM GB/s (% of 8 TB/s), bs16 kv≈68K fp8, 1 GPU"
PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8, help="distinct layer caches cycled per step")
    ap.add_argument("--variant", default="shared", choices=["shared", "unshared", "blocked"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the extra timing lines")
    ap.add_argument("--cpu-requests", type=int, default=2, help="requests in the oracle sample")
    return ap.parse_args()


def make_layers(n_layers, variant, dev):
    import torch

    import workloads

    base = workloads.c16(dev, variant)
    layers = [base]
    for k in range(1, n_layers):
        pool = workloads._fill_values(tuple(base.kv_pool.shape), 0.5, "fp8", 2000 + 100 * k + 1, dev)
        q = workloads._fill_values(tuple(base.q.shape), 1.0, "fp8", 2000 + 100 * k + 2, dev,
                                   chunk_rows=1 << 12)
        q[:, base.real_heads:, :] = torch.zeros((), dtype=q.dtype, device=dev)
        layers.append(workloads.Workload(**{**base.__dict__, "kv_pool": pool, "q": q,
                                            "name": f"{base.name}-layer{k}"}))
    return layers


def time_calls(calls, steps, warmup):
    """Wall time per call over `steps` calls and per-call HIP-event durations."""
    import torch

    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        calls[i % len(calls)]()
        ends[i].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ev = [s.elapsed_time(e) * 1e-3 for s, e in zip(starts, ends)]
    return wall, ev


def cpu_baseline(w, n_req):
    """The float64 oracle on `n_req` full-length requests of the same call."""
    import numpy as np

    from oracle import io as oio

    try:
        from threadpoolctl import threadpool_info

        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    reqs = list(range(n_req))
    args = oio.workload_args(w, reqs)
    t0 = time.perf_counter()
    reps = 0
    while True:
        oio.call_decode(args)
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 3:
            break
    per_sample = (time.perf_counter() - t0) / reps
    per_call = per_sample * w.batch / n_req
    return per_call, cores, f"{n_req} of {w.batch} requests (all {sum(w.lengths[:n_req])} KV rows, 16 heads), {reps} reps; scaled x{w.batch / n_req:g} to one call"


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {a.gpus} is not supported "
              "(multi-GPU sharding is design-only)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mla_latent_attention_amd as mla
    from workloads import accounting

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = make_layers(a.layers, a.variant, dev)
    w0 = layers[0]
    nbytes = accounting.workload_bytes(w0)
    flops = accounting.workload_flops(w0)
    T, H = w0.num_tokens, w0.num_heads
    o = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mla.workspace_bytes(w0.batch, T, H, 1), dtype=torch.uint8, device=dev)

    def call_for(w):
        return lambda: mla.decode(w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                  w.kv_last_page_lens, w.sm_scale, w.q_scale, w.kv_scale,
                                  o=o, max_seqlen_q=1, workspace=ws)

    calls = [call_for(w) for w in layers]
    wall, ev = time_calls(calls, a.steps, a.warmup)
    ev_mean = float(np.mean(ev))
    us = wall * 1e6
    value = nbytes / wall / 1e9
    achieved = nbytes / ev_mean / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(wall * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {
            "workload": f"c16 decode, {a.variant} prefix: batch 16, 16 heads (12 real + 4 zero), "
                        f"qlen 1, kv {min(w0.lengths)}-{max(w0.lengths)} (63,911 shared-prefix slots), "
                        f"fp8 e4m3 pool 5,283,840 x 576, {a.layers} layer caches cycled",
            "global_batch": w0.batch,
            "seq_len": int(np.mean(w0.lengths)),
            "kv_rows_per_call": w0.total_kv,
            "layers_cycled": a.layers,
            "parallelism": "single GPU",
        },
        "us_per_call": round(us, 2),
        "pct_of_8TBs": round(100 * value / PEAK_GBS, 2),
        "algorithmic_bytes_per_call": nbytes,
        "flops_per_call": flops,
        "event_us_per_call": {"mean": round(ev_mean * 1e6, 2),
                              "p10": round(float(np.percentile(ev, 10)) * 1e6, 2),
                              "median": round(float(np.median(ev)) * 1e6, 2),
                              "p90": round(float(np.percentile(ev, 90)) * 1e6, 2)},
        "roofline": {
            "bound": "hbm",
            "kernel": "mla_decode call (decode kernel + split combine kernel)",
            "achieved": round(achieved, 2),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": None,
        },
    }
    if not a.no_variants:
        variants = {}
        wall1, ev1 = time_calls(calls[:1], max(20, a.steps // 4), 5)
        variants["same_layer_back_to_back"] = {"us_per_call": round(wall1 * 1e6, 2),
                                               "GB_s": round(nbytes / wall1 / 1e9, 2)}
        out["variants"] = variants
    if not a.no_cpu_baseline:
        per_call, cores, sample = cpu_baseline(w0, a.cpu_requests)
        out["cpu_baseline"] = {"value": round(nbytes / per_call / 1e9, 4), "unit": "GB/s",
                               "us_per_call": round(per_call * 1e6, 1), "cores": cores,
                               "kind": "oracle", "sample": sample}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

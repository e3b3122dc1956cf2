"""Benchmark: latent MLA decode on one MI355X, batch 16 at kv ~68,430, fp8.

One step = one mla_decode call (plan, index fetch, row gather, QK^T, online
softmax, P.V, split epilogue and combine) over one layer's inputs.  As in a
model step, consecutive steps cycle through `--layers` independent layer
caches (same requests and index lists, separate pools and queries), so a
layer's distinct rows have left the last-level cache before that layer comes
round again.  Inputs are resident in HBM before timing starts.

The calls are captured once in a HIP graph (as a serving loop would) and the
graph is replayed, so the timing is the GPU's, not the Python binding's; the
eager per-call time is reported beside it.

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
CONFIG_NAMES = ("c24_batch24_fp8", "mixed_batch64_fp8", "mixed_batch64_bf16",
                "dcp_local_96heads_qlen4_fp8", "dcp_share_96heads_qlen4_fp8",
                "dcp_share_96heads_qlen4_fp8_f32out", "c16_shared_prefix_cascade_fp8",
                "c16_shared_prefix_cascade_fp8_12heads", "c32_shared_prefix_cascade_fp8_12_vs_16",
                "merge_8_shards_fp32", "merge_8_shards_bf16", "c16_layer_step_rope_decode_v")
PEAK_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0  # dense fp8 MFMA (the decode's Q.K and P.V run on fp8 MFMA)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--layers", type=int, default=8, help="distinct layer caches cycled per step")
    ap.add_argument("--variant", default="shared",
                    choices=["shared", "unshared", "blocked", "paged128", "paged128_unshared"],
                    help="index layout of the timed call (paged128*: mla_decode_paged with "
                         "128-slot pages, the prefix's pages shared or not)")
    ap.add_argument("--eager", action="store_true", help="time eager calls instead of graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the extra timing lines")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations (c24, mixed fp8/bf16, DCP share, merge)")
    ap.add_argument("--only", default=None, choices=sorted(CONFIG_NAMES),
                    help="time just this other configuration and print its line (for profiling)")
    ap.add_argument("--cpu-requests", type=int, default=2, help="requests in the oracle sample")
    ap.add_argument("--no-cpu-runs", action="store_true",
                    help="skip the oracle runs at 1 thread / all threads on the tiny, batch-16 and "
                         "DCP-share samples")
    ap.add_argument("--oracle-timing", default=None, metavar="NPZ",
                    help="(child mode) time the float64 oracle on saved arguments and print JSON")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain fp32 copy-like kernel (out = -in) over BYTES, "
                         "to calibrate HBM byte counters, and exit")
    return ap.parse_args()


def calibrate_copy(nbytes, steps):
    """A plain elementwise kernel reading and writing exactly nbytes each."""
    import torch

    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n * 4, "bytes_written": n * 4, "launches": steps}),
          flush=True)


def make_layers(n_layers, variant, dev):
    """n_layers decode calls over the same requests with separate pools and q."""
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


def with_indices(layers, variant, dev):
    """The same layers with another variant's index lists."""
    import workloads

    shared = 0 if variant == "unshared" else workloads.SHARED_PREFIX
    layout = "blocked" if variant == "blocked" else "random"
    idx = workloads.make_indices(layers[0].lengths, shared, layers[0].kv_pool.shape[0], layout,
                                 2000 + 3, dev, workloads.INDEX_BUFFER)
    return [workloads.Workload(**{**w.__dict__, "kv_indices": idx}) for w in layers]


def with_pages(layers, page_size, dev, shared=True):
    """The same layers as a paged call: a page table of page_size-slot pages
    (the prefix's whole pages shared, or none with shared=False; the rest of
    each request in its own pages)."""
    import workloads

    kvp, idx, last = workloads.make_paged_indices(layers[0].lengths, page_size,
                                                  workloads.SHARED_PREFIX if shared else 0,
                                                  layers[0].kv_pool.shape[0], 2000 + 3, dev)
    return [workloads.Workload(**{**w.__dict__, "kv_indptr": kvp, "kv_indices": idx,
                                  "kv_last_page_lens": last, "page_size": page_size})
            for w in layers]


def extra_layers(base, n_layers, kv_std, seed0, dev):
    """base plus n_layers - 1 copies with separate pools and q (same indices)."""
    import torch

    import workloads

    layers = [base]
    for k in range(1, n_layers):
        pool = workloads._fill_values(tuple(base.kv_pool.shape), kv_std, base.dtype,
                                      seed0 + 100 * k + 1, dev)
        q = workloads._fill_values(tuple(base.q.shape), 1.0, base.dtype, seed0 + 100 * k + 2, dev,
                                   chunk_rows=1 << 12)
        if base.real_heads < base.num_heads:
            q[:, base.real_heads:, :] = torch.zeros((), dtype=q.dtype, device=dev)
        layers.append(workloads.Workload(**{**base.__dict__, "kv_pool": pool, "q": q,
                                            "name": f"{base.name}-layer{k}"}))
    return layers


def config_lines(mla, dev, steps, warmup, n_layers=4, only=None):
    """Time the other decode configurations and the shard merge, each cycling
    n_layers independent inputs under graph replay (only: just that one)."""
    import torch

    import workloads
    from workloads import accounting

    out = {}
    cases = [
        ("c24_batch24_fp8", lambda: workloads.c24(dev), 0.5, torch.bfloat16),
        ("mixed_batch64_fp8", lambda: workloads.mixed(dev, "fp8"), 1.0, torch.bfloat16),
        ("mixed_batch64_bf16", lambda: workloads.mixed(dev, "bf16"), 1.0, torch.bfloat16),
        ("dcp_local_96heads_qlen4_fp8", lambda: workloads.dcp_local(dev), 0.5, torch.bfloat16),
        ("dcp_share_96heads_qlen4_fp8", lambda: workloads.dcp_share(dev), 0.5, torch.bfloat16),
        ("dcp_share_96heads_qlen4_fp8_f32out", lambda: workloads.dcp_share(dev), 0.5,
         torch.float32),
    ]
    for name, make, std, o_dtype in cases:
        if only is not None and name != only:
            continue
        base = make()
        layers = extra_layers(base, n_layers, std, 7000, dev)
        T, H = base.num_tokens, base.num_heads
        o = torch.empty((T, H, 512), dtype=o_dtype, device=dev)
        lse = torch.empty((T, H), dtype=torch.float32, device=dev) if base.return_lse else None
        ws = mla.new_workspace(mla.workspace_bytes(base.batch, T, H, base.max_seqlen_q), dev)

        def call_for(w):
            if w.g_kv_indptr is not None:  # one DCP shard
                return lambda: mla.decode_dcp(
                    w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_lens,
                    w.sm_scale, w.q_scale, w.kv_scale, return_lse=w.return_lse,
                    g_kv_indptr=w.g_kv_indptr, cp_world_size=w.cp_size, cp_rank=w.cp_rank,
                    o_dtype=o_dtype, o=o, lse=lse, max_seqlen_q=w.max_seqlen_q, workspace=ws)
            return lambda: mla.decode(w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                      w.kv_last_page_lens, w.sm_scale, w.q_scale, w.kv_scale,
                                      return_lse=w.return_lse, o=o, lse=lse,
                                      max_seqlen_q=w.max_seqlen_q, workspace=ws)

        wall, ev, n = time_graph([call_for(w) for w in layers], steps, warmup)
        nbytes = accounting.workload_bytes(base)
        flops = accounting.workload_flops(base)
        out[name] = {"us_per_call": round(wall * 1e6, 2), "event_us": stats_us(ev),
                     "GB_s": round(nbytes / wall / 1e9, 2),
                     "pct_of_8TBs": round(100 * nbytes / wall / 1e9 / PEAK_GBS, 2),
                     "TFLOP_s": round(flops / wall / 1e12, 2),
                     "pct_of_fp8_peak": round(100 * flops / wall / 1e12 / PEAK_FP8_TFLOPS, 2),
                     "algorithmic_bytes_per_call": nbytes, "flops_per_call": flops,
                     "kv_rows": base.total_kv, "dtype": base.dtype,
                     "o_dtype": str(o_dtype).replace("torch.", ""), "calls": n}
        del layers, base, o, lse, ws
        torch.cuda.empty_cache()
    for name, heads in (("c16_shared_prefix_cascade_fp8", None),
                        ("c16_shared_prefix_cascade_fp8_12heads", 12)):
        if only is not None and only != name:
            continue
        # The headline call through decode_cascade: the 63,911 shared entries
        # given once, each request's own entries as its suffix; with 12 heads
        # the real heads are passed unpadded (q (16, 12, 576)).
        base = workloads.c16(dev, "shared")
        layers = extra_layers(base, n_layers, 0.5, 7000, dev)
        if heads is not None:
            layers = [workloads.Workload(**{**w.__dict__, "q": w.q[:, :heads].contiguous(),
                                            "num_heads": heads}) for w in layers]
        pre, sptr, suf = workloads.split_prefix(base, workloads.SHARED_PREFIX)
        T, H = base.num_tokens, layers[0].num_heads
        o = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
        ws = mla.new_workspace(mla.cascade_workspace_bytes(base.batch, T, H, 1), dev)

        def cascade_for(w):
            return lambda: mla.decode_cascade(w.q, w.kv_pool, w.qo_indptr, pre, sptr, suf,
                                              w.sm_scale, w.q_scale, w.kv_scale, o=o,
                                              max_seqlen_q=1, workspace=ws)

        wall, ev, n = time_graph([cascade_for(w) for w in layers], steps, warmup)
        nbytes = accounting.workload_bytes(base)
        unique = accounting.cascade_bytes(base, workloads.SHARED_PREFIX)
        out[name] = {"us_per_call": round(wall * 1e6, 2), "event_us": stats_us(ev),
                     "GB_s_effective": round(nbytes / wall / 1e9, 2),
                     "algorithmic_bytes_per_call": nbytes,
                     "cascade_bytes_per_call": unique,
                     "GB_s_cascade_bytes": round(unique / wall / 1e9, 2),
                     "TFLOP_s": round(accounting.workload_flops(base) / wall / 1e12, 2),
                     "pct_of_fp8_peak": round(100 * accounting.workload_flops(base) / wall / 1e12
                                              / PEAK_FP8_TFLOPS, 2),
                     "heads": H, "kv_rows": base.total_kv, "dtype": "fp8", "calls": n}
        del layers, base, o, ws, pre, sptr, suf
        torch.cuda.empty_cache()
    name = "c32_shared_prefix_cascade_fp8_12_vs_16"
    if only is None or only == name:
        # Batch 32 through decode_cascade with the 12 real heads padded to 16
        # and unpadded: the prefix pass's 32 x 12 query rows fill 3 units of
        # 128 rows, the padded 32 x 16 fill 4.
        base = workloads.c32(dev)
        pre, sptr, suf = workloads.split_prefix(base, workloads.SHARED_PREFIX)
        T = base.num_tokens
        res = {}
        for heads in (16, 12):
            layers = extra_layers(base, n_layers, 0.5, 7500, dev)
            if heads == 12:
                layers = [workloads.Workload(**{**w.__dict__, "q": w.q[:, :12].contiguous(),
                                                "num_heads": 12}) for w in layers]
            o = torch.empty((T, heads, 512), dtype=torch.bfloat16, device=dev)
            ws = mla.new_workspace(mla.cascade_workspace_bytes(base.batch, T, heads, 1), dev)
            calls = [(lambda w=w: mla.decode_cascade(w.q, w.kv_pool, w.qo_indptr, pre, sptr, suf,
                                                     w.sm_scale, w.q_scale, w.kv_scale, o=o,
                                                     max_seqlen_q=1, workspace=ws))
                     for w in layers]
            wall, ev, n = time_graph(calls, steps, warmup)
            res[f"heads_{heads}"] = {"us_per_call": round(wall * 1e6, 2), "event_us": stats_us(ev),
                                     "calls": n}
            del layers, o, ws, calls
        res["kv_rows"] = base.total_kv
        res["workload"] = ("batch 32, kv ~68,430, shared 63,911-entry prefix, fp8, through "
                           "mla_decode_cascade: heads_16 = 12 real heads padded with 4 zero heads, "
                           "heads_12 = the 12 real heads unpadded")
        out[name] = res
        del base, pre, sptr, suf
        torch.cuda.empty_cache()
    for parts_dtype in ("fp32", "bf16"):
        if only is not None and only != f"merge_8_shards_{parts_dtype}":
            continue
        sets = [workloads.merge_shards(parts_dtype=parts_dtype, seed=5100 + k, device=dev)
                for k in range(8)]
        o = torch.empty((32, 96, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((32, 96), dtype=torch.float32, device=dev)
        calls = [(lambda op=op, lp=lp: mla.merge_partials(op, lp, o=o, lse=lse))
                 for op, lp in sets]
        wall, ev, n = time_graph(calls, steps, warmup, per_graph=8)
        nbytes = accounting.merge_bytes(8, 32, 96, parts_dtype)
        out[f"merge_8_shards_{parts_dtype}"] = {
            "us_per_call": round(wall * 1e6, 2), "event_us": stats_us(ev),
            "GB_s": round(nbytes / wall / 1e9, 2),
            "pct_of_8TBs": round(100 * nbytes / wall / 1e9 / PEAK_GBS, 2),
            "algorithmic_bytes_per_call": nbytes, "calls": n}
        del sets
    if only is None or only == "c16_layer_step_rope_decode_v":
        out["c16_layer_step_rope_decode_v"] = layer_step_line(mla, dev, steps, warmup)
    return out


def layer_step_line(mla, dev, steps, warmup, n_layers=4):
    """The batch-16 call with the steps either side: the fused rope / fp8 /
    cache-write step, the decode, and the latent -> v_head_dim GEMM, per
    layer (n_layers caches and weights cycled); each step also alone."""
    import torch

    import workloads
    from workloads import accounting

    layers = make_layers(n_layers, "shared", dev)
    w0 = layers[0]
    T, Hp, H = w0.num_tokens, w0.num_heads, w0.real_heads
    sur = [workloads.surround(T, H, 73_728, w0.kv_pool.shape[0], seed=8000 + k, device=dev)
           for k in range(n_layers)]
    kvp = w0.kv_indptr.cpu().tolist()
    # each request's new entry goes to the last slot of its list
    slots = torch.stack([w0.kv_indices[kvp[b + 1] - 1] for b in range(w0.batch)]).to(torch.int32)
    q = torch.empty((T, Hp, 576), dtype=torch.float8_e4m3fn, device=dev)
    o = torch.empty((T, Hp, 512), dtype=torch.bfloat16, device=dev)
    v = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    ws = mla.new_workspace(mla.workspace_bytes(w0.batch, T, Hp, 1), dev)

    def rope(w, s):
        return lambda: mla.rope_quant_cache(s.q_latent, s.q_pe, s.k_latent, s.k_pe, s.positions,
                                            s.cos_sin, w.kv_pool, slots, num_heads_pad=Hp,
                                            q_scale=w.q_scale, kv_scale=w.kv_scale, q_out=q)

    def dec(w):
        return lambda: mla.decode(q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                  w.kv_last_page_lens, w.sm_scale, w.q_scale, w.kv_scale, o=o,
                                  max_seqlen_q=1, workspace=ws)

    def bmm(s):
        return lambda: mla.latent_to_v(o, s.w_uv, out=v)

    def step(w, s):
        r, d, b = rope(w, s), dec(w), bmm(s)
        return lambda: (r(), d(), b())

    ws_step = mla.new_workspace(
        mla._lib.lib().mla_decode_step_workspace_bytes(w0.batch, T, Hp, 1), dev)

    def fused(w, s):
        return lambda: mla.decode_step(s.q_latent, s.q_pe, s.k_latent, s.k_pe, s.positions,
                                       s.cos_sin, slots, w.kv_pool, w.qo_indptr, w.kv_indptr,
                                       w.kv_indices, w.sm_scale, s.w_uv, num_heads_pad=Hp,
                                       q_scale=w.q_scale, kv_scale=w.kv_scale, o_latent=o,
                                       out=v, max_seqlen_q=1, workspace=ws_step)

    res = {}
    for name, calls in (("rope_quant_cache", [rope(w, s) for w, s in zip(layers, sur)]),
                        ("latent_to_v", [bmm(s) for s in sur]),
                        ("decode", [dec(w) for w in layers]),
                        ("layer_step", [step(w, s) for w, s in zip(layers, sur)]),
                        ("layer_step_fused", [fused(w, s) for w, s in zip(layers, sur)])):
        wall, ev, n = time_graph(calls, steps, warmup, per_graph=8)
        res[name] = {"us_per_call": round(wall * 1e6, 2), "event_us": stats_us(ev), "calls": n}
    rope_bytes = (T * H * (512 + 64) * 2 + T * 576 * 2 + T * 8 + T * 256
                  + T * Hp * 576 + T * 576)
    bmm_bytes = T * H * 512 * 2 + H * 128 * 512 * 2 + T * H * 128 * 2
    res["rope_quant_cache"]["algorithmic_bytes_per_call"] = rope_bytes
    res["latent_to_v"]["algorithmic_bytes_per_call"] = bmm_bytes
    res["latent_to_v"]["GB_s"] = round(bmm_bytes / (res["latent_to_v"]["us_per_call"] * 1e-6) / 1e9, 2)
    res["layer_step"]["decode_bytes_per_call"] = accounting.workload_bytes(w0)
    res["layer_step_fused"]["over_decode_us"] = round(
        res["layer_step_fused"]["us_per_call"] - res["decode"]["us_per_call"], 2)
    res["layer_step"]["over_decode_us"] = round(
        res["layer_step"]["us_per_call"] - res["decode"]["us_per_call"], 2)
    res["workload"] = (f"c16 (T={T}, {H} heads padded to {Hp}): rope + fp8 + cache write of the new "
                       f"entries, the decode, then o (T,{H},512) x W_uv ({H},128,512); "
                       f"layer_step: three calls (mla_rope_quant_cache, mla_decode, "
                       f"mla_latent_to_v); layer_step_fused: mla_decode_step (two launches)")
    del layers, sur
    torch.cuda.empty_cache()
    return res


def make_calls(mla, layers, o, ws):
    def call_for(w):
        if w.page_size > 1:
            return lambda: mla.decode_paged(w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                            w.kv_last_page_lens, w.sm_scale, w.q_scale,
                                            w.kv_scale, page_size=w.page_size, o=o,
                                            max_seqlen_q=1, workspace=ws)
        return lambda: mla.decode(w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                  w.kv_last_page_lens, w.sm_scale, w.q_scale, w.kv_scale,
                                  o=o, max_seqlen_q=1, workspace=ws)

    return [call_for(w) for w in layers]


def graph_width(steps, most=8):
    """Calls per captured graph: the largest divisor of `steps` up to `most`,
    so that whole graphs make exactly `steps` calls."""
    return max(d for d in range(1, most + 1) if steps % d == 0)


def time_graph(calls, steps, warmup, per_graph=None):
    """Capture the calls in HIP graphs of `per_graph` consecutive calls each
    (cycling through `calls`; default graph_width(steps)), replay graphs for
    `warmup` calls untimed, then for `steps` calls (exactly, when per_graph
    divides it), with an event on the launch stream between consecutive
    graphs.  Several calls per graph, as in a model step captured whole: a
    graph launch per call leaves a gap of several us between calls that a
    step's own kernels do not have.  Returns (wall s per call over the timed
    calls, per-call event seconds (graph interval / per_graph), calls timed)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    if per_graph is None:
        per_graph = graph_width(steps)
    L = len(calls)
    graphs = []
    for j in range(max(1, -(-L // per_graph))):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(per_graph):
                calls[(j * per_graph + i) % L]()
        graphs.append(g)
    ng = len(graphs)
    reps = max(1, -(-steps // per_graph))
    for i in range(-(-warmup // per_graph)):
        graphs[i % ng].replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(reps):
        graphs[i % ng].replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    n = reps * per_graph
    wall = (time.perf_counter() - t0) / n
    per_call = [ev[i].elapsed_time(ev[i + 1]) * 1e-3 / per_graph for i in range(reps)]
    del graphs
    return wall, per_call, n


def time_eager(calls, steps, warmup):
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
    return wall, ev, steps


def time_cold(calls, steps, mode, flush_bytes=512 << 20):
    """Each call timed alone with HIP events, after a pass over a scratch
    buffer of flush_bytes (outside the events) that evicts the 256 MiB
    last-level cache, as when the other layers of a model step run between two
    calls of a layer.  mode "read" reads the buffer (a sum), so the cache is
    left holding clean lines; mode "write" fills it, so the call first has to
    write back the cache's dirty lines as it evicts them.  Returns the
    per-call event seconds."""
    import torch

    scratch = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    scratch.fill_(1.0)
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def flush(i):
        if mode == "read":
            torch.sum(scratch, dim=0, out=sink)
        else:
            scratch.fill_(float(i & 7))

    for i in range(2):
        flush(i)
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        flush(i)
        starts[i].record()
        calls[i % len(calls)]()
        ends[i].record()
    torch.cuda.synchronize()
    ev = [s.elapsed_time(e) * 1e-3 for s, e in zip(starts, ends)]
    del scratch, sink
    return ev


def cpu_baseline(w, n_req, gpu_out=None):
    """The float64 oracle on `n_req` full-length requests of the same call.
    gpu_out = (o, lse) of the same call on the GPU: its error against the
    oracle on those requests is returned too (max abs and row-relative on o,
    max abs on lse)."""
    import numpy as np

    from oracle import io as oio

    try:
        from threadpoolctl import threadpool_info

        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    args = oio.workload_args(w, list(range(n_req)))
    t0 = time.perf_counter()
    reps = 0
    while True:
        ref = oio.call_decode(args)
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 3:
            break
    per_sample = (time.perf_counter() - t0) / reps
    per_call = per_sample * w.batch / n_req
    rows = sum(w.lengths[:n_req])
    sample = (f"{n_req} of {w.batch} requests ({rows} KV rows x 16 heads), {reps} reps; "
              f"scaled x{w.batch / n_req:g} to one call")
    parity = None
    if gpu_out is not None:
        o_ref, lse_ref = ref
        toks = args["tokens"]
        o = gpu_out[0][toks].float().cpu().numpy().astype(np.float64)
        lse = gpu_out[1][toks].cpu().numpy().astype(np.float64)
        err = np.abs(o - o_ref)
        ref_row = np.abs(o_ref).max(axis=-1)
        live = ref_row > 0
        parity = {"tokens": int(len(toks)), "max_abs": float(err.max()),
                  "row_rel": float((err.max(axis=-1)[live] / ref_row[live]).max()),
                  "lse_abs": float(np.abs(lse - lse_ref).max()),
                  "gate": "max_abs <= 1e-2, row_rel <= 2^-7, lse_abs <= 1e-3"}
    return per_call, cores, sample, parity


def oracle_timing_child(path):
    """Child-process mode: the oracle on saved arguments, with the BLAS thread
    count its environment sets (numpy is imported here, after that is set)."""
    import numpy as np

    from oracle import mla as omla

    with np.load(path, allow_pickle=False) as d:
        args = {k: (d[k].item() if d[k].ndim == 0 else d[k]) for k in d.files}
    try:
        from threadpoolctl import threadpool_info

        info = threadpool_info()
        threads = max([int(i.get("num_threads", 1)) for i in info] or [1])
        blas = ",".join(sorted({f"{i.get('internal_api')}" for i in info})) or "none"
    except Exception:  # pragma: no cover
        threads, blas = -1, "unknown"
    t0 = time.perf_counter()
    reps = 0
    while True:
        omla.mla_decode(**args)
        reps += 1
        if time.perf_counter() - t0 > 5.0 or reps >= 5:
            break
    print(json.dumps({"s_per_call": (time.perf_counter() - t0) / reps, "reps": reps,
                      "threads": threads, "blas": blas}), flush=True)


def cpu_baseline_runs(dev, w16, n_req):
    """The oracle at 1 thread and at all the host's threads, in child processes
    (the thread count must be set before numpy loads), on the tiny call, a
    sample of the batch-16 call and a sample of the DCP share."""
    import subprocess
    import tempfile

    import numpy as np

    import workloads
    from oracle import io as oio
    from workloads import accounting

    cores = len(os.sched_getaffinity(0))
    cases = []
    w = workloads.tiny(dev)
    cases.append(("tiny", w, None, 1.0, accounting.workload_bytes(w), "the whole call"))
    cases.append(("c16_batch16", w16, list(range(n_req)), w16.batch / n_req,
                  accounting.workload_bytes(w16),
                  f"{n_req} of {w16.batch} requests, scaled x{w16.batch / n_req:g}"))
    w5 = workloads.dcp_share(dev)
    cases.append(("dcp_share", w5, [0], float(w5.batch), accounting.workload_bytes(w5),
                  f"1 of {w5.batch} requests, scaled x{w5.batch}"))
    runs = []
    with tempfile.TemporaryDirectory() as tmp:
        for name, w, reqs, scale, nbytes, sample in cases:
            args = oio.workload_args(w, reqs)
            args.pop("tokens")
            path = os.path.join(tmp, f"{name}.npz")
            np.savez(path, **{k: np.asarray(v) for k, v in args.items()})
            for threads in (1, cores):
                env = dict(os.environ, OMP_NUM_THREADS=str(threads),
                           OPENBLAS_NUM_THREADS=str(threads), MKL_NUM_THREADS=str(threads))
                r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-timing",
                                    path], env=env, capture_output=True, text=True, timeout=600)
                if r.returncode != 0:
                    raise RuntimeError(f"oracle timing child failed: {r.stderr[-2000:]}")
                res = json.loads(r.stdout.strip().splitlines()[-1])
                per_call = res["s_per_call"] * scale
                runs.append({"config": name, "threads": res["threads"], "blas": res["blas"],
                             "us_per_call": round(per_call * 1e6, 1),
                             "GB_s": round(nbytes / per_call / 1e9, 5), "sample": sample,
                             "reps": res["reps"]})
    del w5
    return runs, cores


def measured_traffic(variant):
    """HBM bytes per call from the committed counter runs, if they were taken on
    this exact kernel source and workload variant; else None."""
    import hashlib

    try:
        with open(os.path.join(ROOT, "profiles", "traffic_c16.json")) as f:
            rec = json.load(f)
        for path, want in rec["kernel_sources_sha256"].items():
            with open(os.path.join(ROOT, path), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != want:
                    return None
        v = rec["variants"][variant]
        return int(v["fetch_bytes_per_call"]) + int(v["write_bytes_per_call"])
    except (OSError, KeyError, ValueError, AttributeError, TypeError):
        return None


def stats_us(ev):
    import numpy as np

    return {"mean": round(float(np.mean(ev)) * 1e6, 2),
            "p10": round(float(np.percentile(ev, 10)) * 1e6, 2),
            "median": round(float(np.median(ev)) * 1e6, 2),
            "p90": round(float(np.percentile(ev, 90)) * 1e6, 2)}


def main():
    a = parse()
    if a.oracle_timing:
        oracle_timing_child(a.oracle_timing)
        return
    if a.calibrate_copy:
        calibrate_copy(a.calibrate_copy, max(1, a.steps))
        return
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
    if a.only:
        line = config_lines(mla, dev, max(64, a.steps // 4), 8, only=a.only)
        print(json.dumps({"config_only": a.only, **line[a.only]}), flush=True)
        return
    if a.variant.startswith("paged128"):
        layers = with_pages(make_layers(a.layers, "shared", dev), 128, dev,
                            shared=a.variant == "paged128")
    else:
        layers = make_layers(a.layers, a.variant, dev)
    w0 = layers[0]
    nbytes = accounting.workload_bytes(w0)
    flops = accounting.workload_flops(w0)
    T, H = w0.num_tokens, w0.num_heads
    o = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    ws = mla.new_workspace(mla.workspace_bytes(w0.batch, T, H, 1), dev)
    calls = make_calls(mla, layers, o, ws)
    timer = time_eager if a.eager else time_graph
    wall, ev, steps = timer(calls, a.steps, a.warmup)
    ev_mean = float(np.mean(ev))
    value = nbytes / wall / 1e9
    achieved = nbytes / ev_mean / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
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
                        f"fp8 e4m3 pool 5,283,840 x 576, {a.layers} layer caches cycled, "
                        f"{'eager calls' if a.eager else 'HIP graph replay'}",
            "global_batch": w0.batch,
            "seq_len": int(np.mean(w0.lengths)),
            "kv_rows_per_call": w0.total_kv,
            "layers_cycled": a.layers,
            "parallelism": "single GPU",
        },
        "us_per_call": round(wall * 1e6, 2),
        "pct_of_8TBs": round(100 * value / PEAK_GBS, 2),
        "algorithmic_bytes_per_call": nbytes,
        "flops_per_call": flops,
        "event_us_per_call": stats_us(ev),
        "roofline": {
            "bound": "hbm",
            "kernel": ("mla_decode call: " + ("mla_decode_fp8_paged_kernel" if w0.page_size > 1
                                              else "mla_decode_fp8_kernel")
                       + " + mla_combine_kernel"),
            "achieved": round(achieved, 2),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": measured_traffic(a.variant) if a.layers == 8 else None,
        },
    }
    if not a.no_variants:
        variants = {}
        wall1, ev1, _ = timer(calls[:1] * 4, max(16, a.steps // 8), 4)
        variants["same_layer_back_to_back"] = {"us_per_call": round(wall1 * 1e6, 2),
                                               "GB_s": round(nbytes / wall1 / 1e9, 2)}
        if not a.eager:
            wall_e, ev_e, _ = time_eager(calls, max(16, a.steps // 4), 4)
            variants["eager_calls_incl_host_overhead"] = {"us_per_call": round(wall_e * 1e6, 2),
                                                          "event_us": stats_us(ev_e)}
        # Cold (the survey's protocol): every call timed alone after a pass
        # over 512 MiB that evicts the 256 MiB last-level cache; per-call
        # events, median.
        for mode in ("read", "write"):
            st_c = stats_us(time_cold(calls, 32, mode))
            med_c = st_c["median"] * 1e-6
            variants[f"cold_after_512MiB_{mode}"] = {
                "us_per_call": st_c["median"], "event_us": st_c,
                "GB_s": round(nbytes / med_c / 1e9, 2),
                "pct_of_8TBs": round(100 * nbytes / med_c / 1e9 / PEAK_GBS, 2)}
        for var in ("unshared", "blocked"):
            if var == a.variant:
                continue
            vcalls = make_calls(mla, with_indices(layers, var, dev), o, ws)
            wv, evv, _ = timer(vcalls, max(16, a.steps // 4), a.warmup)
            variants[f"{var}_prefix"] = {"us_per_call": round(wv * 1e6, 2),
                                         "GB_s": round(nbytes / wv / 1e9, 2),
                                         "pct_of_8TBs": round(100 * nbytes / wv / 1e9 / PEAK_GBS, 2)}
        # The same call through mla_decode_paged with 128-slot pages (one index
        # per page instead of one per entry).
        for name, shared in (("paged128", True), ("paged128_unshared_prefix", False)):
            paged = with_pages(layers, 128, dev, shared)
            pbytes = accounting.workload_bytes(paged[0])
            wp, evp, _ = timer(make_calls(mla, paged, o, ws), max(16, a.steps // 4), a.warmup)
            variants[name] = {"us_per_call": round(wp * 1e6, 2),
                              "algorithmic_bytes_per_call": pbytes,
                              "GB_s": round(pbytes / wp / 1e9, 2),
                              "pct_of_8TBs": round(100 * pbytes / wp / 1e9 / PEAK_GBS, 2)}
            del paged
        out["variants"] = variants
    if not a.no_configs:
        del calls, layers
        torch.cuda.empty_cache()
        out["configs"] = config_lines(mla, dev, max(64, a.steps // 4), 8)
    if not a.no_cpu_baseline and w0.page_size == 1:
        o_chk, lse_chk = mla.decode(w0.q, w0.kv_pool, w0.qo_indptr, w0.kv_indptr, w0.kv_indices,
                                    w0.kv_last_page_lens, w0.sm_scale, w0.q_scale, w0.kv_scale,
                                    return_lse=True, max_seqlen_q=1)
        torch.cuda.synchronize()
        per_call, cores, sample, parity = cpu_baseline(w0, a.cpu_requests, (o_chk, lse_chk))
        out["cpu_baseline"] = {"value": round(nbytes / per_call / 1e9, 4), "unit": "GB/s",
                               "us_per_call": round(per_call * 1e6, 1), "cores": cores,
                               "kind": "oracle", "sample": sample}
        out["parity_vs_oracle"] = parity
        if not a.no_cpu_runs:
            runs, host_cores = cpu_baseline_runs(dev, w0, a.cpu_requests)
            out["cpu_baseline"]["runs"] = runs
            out["cpu_baseline"]["host_cores"] = host_cores
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

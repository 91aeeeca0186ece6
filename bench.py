"""Benchmark: RESOLVE + top-k sparse attention per decode layer on one MI355X.

Workload (default): batch 8 requests, 1 layer, context 131072 each, MLA-style
576-element bf16 latent records shared by 64 query heads, k = 2048 selected
positions, B = 4096 buffer slots, synthetic 13% Zipf(1.1)-recency drift
traces. A step is one decode step: hs_stage_run (the step's selections and
queries copied into fixed device buffers, standing in for the indexer), then
per layer hs_resolve (hash, probe, victim select, in-place update,
host-to-device miss fetch) and hs_sparse_attn (+ split-k combine). One
hipGraph holds the whole step and is replayed for every step with no host
synchronisation. Inputs (pool, every step's selections and queries) are
resident in memory before the timed region.

Prints one JSON line with the time per layer, the duration of each kernel
class (HIP events carrying each dispatch's own start and end times, over
the same steps replayed eagerly), the roofline of the dominant kernel, the
attention kernel's HBM roofline, the miss fetch's host-link rate, and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
HOST_LINK_PEAK_GBS = 63.0      # PCIe Gen5 x16, one direction, nominal
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "resolve+sparse-attn µs/layer at batch 8, k=2048; achieved HBM and host GB/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=120)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", type=int, default=3,
                    help="workload 1..6 (3 = batch-8 MLA; 6 = batch-8 MLA over 8 layers in "
                         "groups of 4 that reuse one selection)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate budget of the CPU oracle baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device-to-device copy four times (the reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--path", choices=("auto", "fused", "split"), default="auto",
                    help="fused: hs_resolve_attn (misses fetched by the attention kernels); "
                         "split: hs_resolve (which also fetches the misses) then "
                         "hs_sparse_attn; auto: fused for MHA records, split for latent "
                         "records (the faster of the two for each on MI355X)")
    ap.add_argument("--gather-bytes", type=int, default=0,
                    help="hs_tuning.gather_bytes_per_lane: bytes of host reads each lane of the "
                         "resolve's miss fetch keeps in flight (16, 32, 64 or 128; 0 = the "
                         "library's choice)")
    ap.add_argument("--fetch", choices=("auto", "inline", "kernel"), default="auto",
                    help="hs_tuning.resolve_fetch: where hs_resolve moves the misses (inline = in "
                         "the resolve kernel, its first host reads overlapping the victim "
                         "selection; kernel = a gather kernel of its own after the resolve, "
                         "whose duration is the gather phase alone; auto = inline for 4 or more "
                         "units per batch)")
    ap.add_argument("--share", choices=("prefetch", "serial", "none"), default="prefetch",
                    help="layer groups that reuse one selection (workload 6): prefetch = one "
                         "resolve per group, the later layers' fetches on a second stream "
                         "overlapping attention; serial = the same on one stream; none = every "
                         "layer resolves on its own")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 256 << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 4}), flush=True)


def host_dma_rate():
    """Pinned host-to-device copy rate (GB/s) of the DMA engines for 2 MB and
    256 MB copies: the practical ceiling of the host link on this machine."""
    import torch
    out = {}
    for mb in (2, 256):
        n = mb << 20
        h = torch.empty(n, dtype=torch.uint8, pin_memory=True)
        d = torch.empty(n, dtype=torch.uint8, device="cuda")
        d.copy_(h, non_blocking=True)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 8 if mb == 2 else 3
        e0.record()
        for _ in range(reps):
            d.copy_(h, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        out[f"{mb}MB"] = round(n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        del h, d
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def attn_bytes(w, n_units):
    """Algorithmic HBM bytes of one attention launch over n_units units:
    the k selected rows read once, the queries read, the outputs written."""
    rows = n_units * w.k * w.rec_bytes
    q = n_units * w.n_q_heads * w.q_dim * (4 if w.q_dtype == 0 else 2)
    out = n_units * w.n_q_heads * w.out_dim * 4
    return rows + q + out


def attn_flops(w, n_units):
    if w.kind == "mha":
        return n_units * 4.0 * w.n_q_heads * w.head_dim * w.k
    return n_units * 2.0 * w.n_q_heads * w.k * (w.q_dim + w.out_dim)


def cpu_baseline(w, traces, budget_s, one_thread_steps=0):
    """The oracle (resolve + fp64 attention) on the first steps of the same
    trace, all units of each step in parallel over the host cores, until
    the time budget is spent; then, if asked, the next few steps on one
    thread. Returns (us per layer-step, steps, threads, us per layer-step on
    one thread or None)."""
    import oracle
    from tiered_kv_cache_hs_amd import inputs as I

    R, L = w.n_requests, w.n_layers
    pools, bufs, lens = {}, {}, {}
    max_steps = traces.shape[0]
    for r in range(R):
        for l in range(L):
            u = r * L + l
            pool = np.zeros((w.capacity(r, max_steps), w.rec_bytes), dtype=np.uint8)
            pos = np.unique(traces[:, u, :].astype(np.int64))
            pos = pos[(pos >= 0) & (pos < w.ctx[r])]
            I.fill_records(w, pool.ctypes.data, r, l, positions=pos)
            pools[u], lens[u] = pool, w.ctx[r]
            bufs[u] = oracle.OracleBuffer(w.B[r], w.rec_bytes, with_rows=True)
    slots = np.empty((R * L, w.k), np.int32)
    miss = np.empty(R * L, np.int32)
    out = np.empty((R * L, w.n_q_heads, w.out_dim), np.float32)
    step_times, threads = [], 1
    one_times = []
    t_start = time.perf_counter()
    for t in range(max_steps):
        q = I.gen_queries(w, t)
        units = []
        for u in range(R * L):
            b = bufs[u]
            x = oracle.OracleUnitC()
            x.B, x.k = b.B, w.k
            x.pos, x.stamp, x.clock = b.pos.ctypes.data, b.stamp.ctypes.data, b.clock.ctypes.data
            x.err, x.rows, x.rec_bytes = b.err.ctypes.data, b.rows.ctypes.data, w.rec_bytes
            x.pool, x.pool_len = pools[u].ctypes.data, lens[u]
            x.topk = traces[t, u].ctypes.data
            x.slots, x.miss = slots[u].ctypes.data, miss[u:].ctypes.data
            x.kind = 0 if w.kind == "mha" else 1
            x.Hq, x.Hkv, x.D, x.Dl, x.Dr = w.n_q_heads, w.n_kv_heads, w.head_dim, w.latent_dim, w.rope_dim
            x.kv_dtype, x.q_dtype, x.sm_scale = w.dtype, w.q_dtype, np.float32(w.sm_scale)
            x.q, x.out = q[u].ctypes.data, out[u].ctypes.data
            units.append(x)
        t0 = time.perf_counter()
        over = len(step_times) >= 2 and time.perf_counter() - t_start > budget_s
        if over or (one_thread_steps and t >= max_steps - one_thread_steps):
            if len(one_times) >= one_thread_steps:
                break
            oracle.step_batch(units, 1)  # the same oracle on one host thread
            one_times.append(time.perf_counter() - t0)
            continue
        threads = oracle.step_batch(units, 0)
        step_times.append(time.perf_counter() - t0)
    # step 0 is the cold all-miss step; report the warm steps when there are any
    warm = step_times[1:] if len(step_times) > 1 else step_times
    one = 1e6 * float(np.median(one_times)) / L if one_times else None
    return 1e6 * float(np.median(warm)) / L, len(step_times), threads, one


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path runs on a "
              "single MI355X; multi-GPU sharding is described in the design notes only)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch

    from tiered_kv_cache_hs_amd import hisparse as H
    from tiered_kv_cache_hs_amd import inputs as I
    from tiered_kv_cache_hs_amd.session import Session

    H.lib()
    fetch_mode = {"auto": 0, "inline": 1, "kernel": 2}[args.fetch]
    H.hs_set_tuning(gather_bytes_per_lane=args.gather_bytes, resolve_fetch=fetch_mode)
    w = I.workload(args.workload)
    W, K = args.warmup, args.steps
    total = W + K
    print(f"[bench] workload {w.name}: building session ({total} steps)", file=sys.stderr, flush=True)
    fill = "full" if w.n_units * max(w.ctx) * w.rec_bytes <= (8 << 30) else "touched"
    fused = args.path == "fused" or (args.path == "auto" and w.kind == "mha")
    sess = Session(w, total, fill=fill, fused=fused, share_mode=args.share)
    fused = fused and not sess.grouped  # a group's resolve is planned apart from attention
    sess.capture()
    print("[bench] step graph captured (one graph, replayed every step)", file=sys.stderr,
          flush=True)

    # ---- timed region: K replays of the one graph (steps W .. W+K-1)
    for t in range(W):
        sess.replay(t)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for t in range(W, total):
        sess.replay(t)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / K
    print(f"[bench] timed {K} steps: {ms_step * 1000:.1f} us/step (wall {wall * 1e3 / K:.3f} ms/step)",
          file=sys.stderr, flush=True)

    # ---- outside the timed region: the whole trace three times from a reset
    # state, an event pair around each replay (per-step spread; step 0, the
    # cold all-miss step, reported on its own)
    reps = []
    for rep in range(3):
        sess.reset()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(total)]
        for t in range(total):
            evs[t][0].record()
            sess.replay(t)
            evs[t][1].record()
        torch.cuda.synchronize()
        reps.append(np.array([a.elapsed_time(b) * 1000.0 / w.n_layers for a, b in evs]))
    per_step = np.median(np.stack(reps), axis=0)
    warm = per_step[1:]
    step_spread = {"cold_step0": round(float(per_step[0]), 2),
                   "p10": round(float(np.percentile(warm, 10)), 2),
                   "median": round(float(np.median(warm)), 2),
                   "p90": round(float(np.percentile(warm, 90)), 2),
                   "median_per_repeat": [round(float(np.median(r[1:])), 2) for r in reps],
                   "unit": "us/layer, one event pair per replayed step, every step of the trace "
                           "3 times from a reset state (per-step median over the repeats)"}
    dma = host_dma_rate()

    # ---- the same steps again from a reset state, eagerly in the graph's
    # form (stage + the step over the fixed buffers), each kernel carrying
    # events that take its dispatch's start and end times
    sess.reset()
    miss_hist = torch.zeros((total, w.n_layers, w.n_requests), dtype=torch.int32, device="cuda")
    for t in range(total):
        if t == W:
            torch.cuda.synchronize()
            H.hs_trace_enable(True)
            H.hs_trace_read()
        sess.staged_step()
        miss_hist[t].copy_(sess.miss)
    tr = H.hs_trace_read()
    H.hs_trace_enable(False)
    # every layer fetches its own records of its resolve's misses (the misses
    # of a layer in a group are those of the group's resolve)
    src = [sess.resolved_layer(l) for l in range(w.n_layers)]
    misses = miss_hist[W:, src, :].cpu().numpy().astype(np.int64)  # [K][L][R]
    per = {c: (tr[c][0] / tr[c][1] if tr[c][1] else 0.0) for c in H.TRACE_CLASSES}

    # units attended per launch, on average (each launch covers one layer's
    # requests)
    attn_launches_per_step = tr["attn"][1] / K if tr["attn"][1] else 1.0
    units_per_launch = w.n_units / attn_launches_per_step
    a_bytes = attn_bytes(w, 1) * units_per_launch
    a_flops = attn_flops(w, 1) * units_per_launch
    attn_us = per["attn"]
    attn_gbs = a_bytes / (attn_us * 1e-6) / 1e9 if attn_us else 0.0
    attn_kernel = "hs_k_attn_latent" if w.kind == "latent" else "hs_k_attn_mha"
    # the kernels that move the misses over the host link: the attention
    # kernel (fused path); else the resolve kernel itself on batches of 4 or
    # more units, the gather kernel on smaller ones, and the gather kernel
    # for the later layers of a group (hs_prefetch). The host-link roofline
    # is that of the class moving the most bytes.
    lead = np.array([src[l] == l for l in range(w.n_layers)])
    lead_bytes = int(misses[:, lead, :].sum()) * w.rec_bytes
    follow_bytes = int(misses[:, ~lead, :].sum()) * w.rec_bytes
    if fused:
        cls_bytes = {"attn": lead_bytes + follow_bytes}
    else:
        cls_bytes = {"resolve": 0, "gather": follow_bytes}
        inline = fetch_mode == 1 or (fetch_mode == 0 and w.n_requests >= 4)
        cls_bytes["resolve" if inline else "gather"] += lead_bytes
    fetch_class = max(cls_bytes, key=cls_bytes.get)
    fetch_us = per[fetch_class]
    miss_bytes_launch = cls_bytes[fetch_class] / max(1, tr[fetch_class][1])
    host_gbs = miss_bytes_launch / (fetch_us * 1e-6) / 1e9 if fetch_us else 0.0
    miss_rate = float(misses.sum()) / (K * w.n_units * w.k)

    roof_attn = {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                 "kernel": attn_kernel, "avg_us": round(attn_us, 2),
                 "bytes_per_launch": int(a_bytes),
                 "tflops": round(a_flops / (attn_us * 1e-6) / 1e12, 2) if attn_us else 0.0}
    roof_host = {"bound": "host_link", "achieved": round(host_gbs, 2),
                 "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                 "frac": round(host_gbs / HOST_LINK_PEAK_GBS, 4), "traffic": None,
                 "kernel": {"attn": attn_kernel, "gather": "hs_k_gather",
                            "resolve": "hs_k_resolve"}[fetch_class], "avg_us": round(fetch_us, 2),
                 "bytes_per_launch": int(miss_bytes_launch)}
    if fused:
        # one kernel moves both; its bound is the resource whose peak-rate
        # time for the launch's bytes is longer
        t_host = miss_bytes_launch / (HOST_LINK_PEAK_GBS * 1e9)
        t_hbm = a_bytes / (HBM_PEAK_GBS * 1e9)
        dominant = roof_host if t_host >= t_hbm else roof_attn
    else:
        dominant = roof_host if fetch_us >= attn_us else roof_attn

    from tiered_kv_cache_hs_amd.profiling import stored_traffic
    dominant["traffic"] = stored_traffic(w.name, dominant["kernel"], args.path)
    roof_attn["traffic"] = stored_traffic(w.name, attn_kernel, args.path)
    result = {
        "metric": METRIC,
        "value": round(ms_step * 1000.0 / w.n_layers, 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == I.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "requests": w.n_requests, "layers": w.n_layers,
                   "context": w.ctx[0] if len(set(w.ctx)) == 1 else "per-request",
                   "k": w.k, "B": w.B[0] if len(set(w.B)) == 1 else "per-request",
                   "q_heads": w.n_q_heads, "record_bytes": w.rec_bytes, "kind": w.kind,
                   "graph": "one hipGraph replayed for every step (selections and queries "
                            "staged into fixed buffers on the device)",
                   "fetch": args.fetch,
                   "path": ("hs_resolve_attn" if fused else "hs_resolve + hs_sparse_attn")
                   + (f" (layer groups of {w.share}: {sess.share_mode})" if sess.grouped else "")},
        "roofline": dominant,
        "roofline_attn": roof_attn,
        "host_link": roof_host,
        "kernels_us": {c: round(per[c], 2) for c in H.TRACE_CLASSES},
        "miss_rate": round(miss_rate, 4),
        "fetch_bytes_by_kernel": {c: int(v / K) for c, v in cls_bytes.items()},
        "miss_bytes_per_step": int(misses.sum() * w.rec_bytes / K),
        "step_spread": step_spread,
        "host_dma_h2d_gbs": dma,
    }
    sess.close()

    if not args.no_cpu:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        # the oracle samples the same trace from its start, as far as the
        # time budget (or the workload's own length) goes
        traces = I.gen_traces(w, max(total, w.steps))
        us, n_steps, threads, us1 = cpu_baseline(w, traces, args.cpu_seconds,
                                                 one_thread_steps=3 if w.n_units <= 8 else 0)
        result["cpu_baseline"] = {
            "value": round(us, 1), "unit": "us/layer", "cores": int(threads), "kind": "oracle",
            "threads_used": int(threads), "nproc": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(),
            "sample": f"first {n_steps} steps of the same trace (step 0 cold, median of the "
                      f"rest), all {w.n_units} units per step, resolve + fp64 attention",
            "single_thread": None if us1 is None else round(us1, 1),
            "single_thread_sample": "the next 3 steps on one host thread (median)"
                                    if us1 is not None else None}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

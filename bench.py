"""Benchmark of the HSTU block forward with a paged KV cache on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C4]

One step is one whole request through the hot path: restore the cache
metadata to its pre-request state, look the batch up, evict least-recently
used users if pages are short, allocate pages, upload the page table and the
request plan, then run every layer (pre-norm, f1 + SiLU, K/V append,
attention over cached + new keys, LayerNorm(AV) * U, f2 + residual) on the
new tokens, and score the candidate rows with the multitask ranking head.  The new-token inputs are already in device memory when timing
starts.  Prints one JSON line: new tokens per second, the dominant kernel
against its roofline (duration from HIP events on its launch stream), and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_PCIE_GBS = 64.0       # host link, per direction

WORKLOAD_TEXT = {
    "C2": "3-layer bf16 HSTU stack, full recompute (no cache): batch 8, d_model 512, 4 heads x 128, "
          "history uniform [1024, 4096] + 64 target-aware candidates per user",
    "C3": "3-layer bf16 HSTU stack, 100% paged-cache hit (32-token pages, permuted placement): batch 8, "
          "d_model 512, 4 heads x 128, cached history uniform [1024, 4096], 64 new candidates per user",
    "C4": "8-layer bf16 HSTU stack, batch 8, d_model 512, 4 heads x 128; history lognormal(median 2048, "
          "sigma 1) clipped to [256, 8192] + 64 candidates; 50% of users hit a paged cache (32-token "
          "pages), the rest prefill and append; the pool forces LRU eviction of stale users",
    "C5": "8-layer bf16 HSTU stack, batch 128, d_model 512, 4 heads x 128; history lognormal(median 2048, "
          "sigma 1) clipped to [128, 16384], 100% paged-cache hit (64-token pages), 256 target-aware "
          "candidates, 128 rab buckets",
}


def attention_bytes(req, H, dh, es=2):
    """Algorithmic HBM bytes of one attention launch: every visible key/value
    row once per (user, head), the queries once, the fp32 output once."""
    kv = 0
    for c, t, T in zip(req.cached_len, req.new_len, req.n_targets):
        if t == 0:
            continue
        kv += int(c + t)
    n = int(sum(req.new_len))
    return kv * H * dh * 2 * es + n * H * dh * (es + 4)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="C4", choices=["C2", "C3", "C4", "C5"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-serving", action="store_true", help="skip the serving-loop latency measurement")
    ap.add_argument("--no-training", action="store_true", help="skip the training-step measurement")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (reference for HBM traffic counters)")
    args = ap.parse_args(argv)
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 3}), flush=True)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch

    from generative_recommender_sequence_amd import hstu, profiling, runtime
    from generative_recommender_sequence_amd.workloads import head_weights, workload_for

    runtime.require_gpu()
    torch.cuda.set_device(0)
    w = workload_for(args.workload, args.seed)
    cfg = w.cfg
    scn = runtime.Scenario(w)
    scn.prefill()
    users, new_len, n_targets, norm_n, rows = scn.request_inputs()
    x = scn._x(rows)                       # new-token inputs resident in HBM
    n_new = int(sum(new_len))

    # size the workspace once for the request shape
    scn.restore()
    req0 = scn.make_request(rows)[0]
    ws = runtime.workspace_for(scn.model, req0)
    info0 = req0.info
    req0.close()

    rbufs = runtime.RequestBuffers(cfg.batch, scn.max_pages, int(info0.meta_bytes) + 4096)
    ybufs = [torch.empty_like(x), torch.empty_like(x)]
    # the multitask ranking head scores every candidate row of the last layer
    head = runtime.Head(head_weights(cfg.d_model, seed=args.seed), scn.dtype)
    cand = torch.from_numpy(runtime.candidate_row_list(new_len, n_targets)).cuda()
    logits = torch.empty((max(cand.numel(), 1), head.tasks), dtype=torch.float32, device="cuda")

    def step():
        scn.restore()
        req = runtime.prepare(scn.cache, users, new_len, n_targets, norm_n, scn.max_pages, cfg.num_heads,
                              cfg.head_dim, bufs=rbufs)
        y = runtime.forward(scn.model, req, x, scn.cache, ws, out_bufs=ybufs)
        head(y, cand, out=logits)
        return req, y

    # W warm-up requests, continued until the GPU has run for at least 0.3 s
    # (clocks and caches settle; none of it is timed)
    pending = []
    t_w = time.perf_counter()
    n_w = 0
    while n_w < args.warmup or time.perf_counter() - t_w < 0.3:
        pending.append(step()[0])
        n_w += 1
        if len(pending) >= 16:
            torch.cuda.synchronize()
            for r in pending:
                r.close()
            pending.clear()
    torch.cuda.synchronize()
    for r in pending:
        r.close()
    pending.clear()

    # timed region: K whole requests, nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        pending.append(step()[0])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = 1000.0 * (t1 - t0) / args.steps
    for r in pending:
        r.close()
    pending.clear()
    # the same K requests again with every kernel bracketed by HIP events on
    # its launch stream: per-kernel durations for the roofline
    hstu.hstu_timing_enable(True)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        pending.append(step()[0])
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    kern = {}
    for name in hstu.TIMED_KERNELS:
        n, ms = hstu.hstu_timing_read(name)
        if n:
            kern[name] = {"launches": n, "avg_us": round(1000.0 * ms / n, 2), "ms_per_step": round(ms / args.steps, 4)}
    hstu.hstu_timing_enable(False)
    ms_instrumented = 1000.0 * (t3 - t2) / args.steps
    req_last = pending[-1]
    for r in pending[:-1]:
        r.close()

    # dominant kernel: attention
    H, dh = cfg.num_heads, cfg.head_dim
    flops = 4.0 * dh * H * float(req_last.info.pairs)
    bytes_ = float(attention_bytes(req_last, H, dh))
    att_us = kern["attention"]["avg_us"]
    cached_frac = float(sum(c for c in req_last.cached_len)) / max(1.0, float(sum(req_last.kv_len)))
    if args.workload in ("C3", "C5"):
        achieved = bytes_ / (att_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        achieved = flops / (att_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None}
    traffic = profiling.read_traffic(args.workload)
    roof["traffic"] = None if traffic is None else round(traffic, 0)
    roof.update({"kernel": "attention (attn_bf16_kernel, paged)", "avg_us": att_us,
                 "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": bytes_,
                 "unmasked_pairs_per_head": int(req_last.info.pairs)})
    req_last.close()

    n_evicted = int(len(scn_evicted(scn, users, new_len)))
    serving_out = None
    if not args.no_serving and args.workload == "C4":
        serving_out = serving_results(w, args.seed)
    training_out = None
    if not args.no_training and args.workload == "C4":
        training_out = training_results(args.seed)
    tier = host_tier_rates(scn) if scn.cache is not None else None   # attaches a host tier: last

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, scn, users, new_len, n_targets, norm_n, rows)

    out = {
        "metric": "HSTU new tokens/s at batch 8, 8 layers, cache hit; % HBM / MFMA roofline",
        "value": round(n_new / (ms_per_step / 1000.0), 1),
        "unit": "new tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_w,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal weights/inputs, random-init; shapes of the pages' benchmark)",
        "config": {"workload": f"{args.workload}: {WORKLOAD_TEXT[args.workload]}", "global_batch": cfg.batch,
                   "layers": cfg.num_layers, "d_model": cfg.d_model, "heads": H, "head_dim": dh,
                   "new_tokens_per_step": n_new,
                   "candidate_tokens_per_step": int(sum(n_targets)),
                   "cached_key_fraction": round(cached_frac, 4),
                   "evicted_users_per_step": n_evicted,
                   "attention_work_items": int(info0.n_work_items),
                   "head": f"{head.tasks} tasks x MLP({cfg.d_model}-{head.hidden}-1) on every candidate row",
                   "seed": args.seed},
        "roofline": roof,
        "kernels": kern,
        "kernel_ms_per_step": round(sum(k["ms_per_step"] for k in kern.values()), 4),
        "ms_per_step_event_instrumented": round(ms_instrumented, 4),
        "candidate_tokens_per_s": round(sum(n_targets) / (ms_per_step / 1000.0), 1),
        "host_tier": tier,
        "serving": serving_out,
        "training": training_out,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def host_tier_rates(scn, reps=3):
    """Host-tier copies outside the timed region: every cached user of the
    pre-request state is offloaded to a pinned host tier that just holds them,
    then onboarded back, `reps` times.  Rate = K and V bytes of every layer of
    the moved pages / the event-timed duration of the call's GPU work (one
    tier-copy launch).  The cache is left with a host tier attached."""
    import torch

    from generative_recommender_sequence_amd import hstu, runtime
    cache, w = scn.cache, scn.w
    scn.restore()
    ids = [int(u) for u, h in zip(w.user_ids, w.hit) if h] + [int(u) for u in w.stale_ids]
    where, lens = hstu.kv_residency(cache.h, ids)
    ids = [u for u, wh in zip(ids, where) if wh == 1]
    pages = sum(-(-int(n) // cache.page_size) for n, wh in zip(lens, where) if wh == 1)
    if not pages:
        return None
    es = 2 if cache.dtype == hstu.HSTU_BF16 else 4
    moved = pages * cache.num_layers * 2 * cache.num_heads * cache.page_size * cache.head_dim * es
    cache.attach_host(pages)
    s = runtime.stream_handle()
    times = {"offload": [], "onboard": []}
    for _ in range(reps):
        for kind in ("offload", "onboard"):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if kind == "offload":
                hstu.kv_offload(cache.h, ids, s)
            else:
                hstu.kv_onboard(cache.h, ids, s)
            e1.record()
            e1.synchronize()
            times[kind].append(e0.elapsed_time(e1))
    out = {"users": len(ids), "pages": pages, "bytes_per_call": moved, "link": "PCIe 5.0 x16",
           "link_peak_GBps_per_direction": PEAK_PCIE_GBS}
    for kind, ts in times.items():
        ms = sorted(ts)[len(ts) // 2]
        out[f"{kind}_ms"] = round(ms, 3)
        out[f"{kind}_GBps"] = round(moved / (ms * 1e-3) / 1e9, 2)
    return out


def training_results(seed, steps=5, warmup=2):
    """One training step of C2's model and batch (3 bf16 layers, batch 8,
    histories uniform [1024, 4096] + 64 candidates, every position computed):
    the forward keeping its taps, then hstu_layer_backward through every
    layer for a seeded dL/dY.  Outside the timed request; inputs resident.
    The backward attention's roofline uses 5 products per visible pair and
    head (S recomputed, dP, dV, dK, dQ: 10 dh FLOPs per pair)."""
    import torch

    from generative_recommender_sequence_amd import hstu, runtime
    from generative_recommender_sequence_amd.workloads import round_bf16, workload_for

    w = workload_for("C2", seed)
    cfg = w.cfg
    scn = runtime.Scenario(w)
    req, x = scn.make_request()
    rng = np.random.default_rng([seed, 0xB3D])
    n = int(sum(req.new_len))
    dy = torch.from_numpy(round_bf16(rng.standard_normal((n, cfg.d_model)).astype(np.float32))).cuda().to(
        torch.bfloat16)
    ws = [None]

    def step():
        y, saved = runtime.forward_for_backward(scn.model, req, x)
        dx, grads = runtime.backward(scn.model, req, saved, dy)
        return dx

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = 1000.0 * (time.perf_counter() - t0) / steps
    hstu.hstu_timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kern = {}
    for name in hstu.TIMED_KERNELS:
        cnt, tot = hstu.hstu_timing_read(name)
        if cnt:
            kern[name] = {"launches": cnt, "ms_per_step": round(tot / steps, 4)}
    hstu.hstu_timing_enable(False)
    pairs = float(req.info.pairs)
    bwd_att_ms = kern["bwd_attention"]["ms_per_step"] / cfg.num_layers
    flops = 10.0 * cfg.head_dim * cfg.num_heads * pairs
    achieved = flops / (bwd_att_ms * 1e-3) / 1e12
    req.close()
    return {"workload": "C2 model and batch: 3 bf16 layers, batch 8, histories uniform [1024, 4096] + 64 "
                        "candidates, forward (with taps) + backward, seeded dL/dY",
            "tokens_per_step": n, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(n / (ms / 1000.0), 1),
            "kernels_ms_per_step": {k: v["ms_per_step"] for k, v in kern.items()},
            "backward_attention_roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                                            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                                            "algorithmic_flops_per_layer": flops,
                                            "ms_per_layer": round(bwd_att_ms, 4)}}


def serving_results(w, seed, users=32):
    """Latency under load of the serving loop (dynamic batches of up to 8,
    500 us batching delay, host cache work overlapped with the previous
    batch): a population of `users` users with the workload's history
    distribution, each request bringing 0-16 new history events and 64
    candidates; the device pool holds about half the population, so misses
    (evicted users) recompute their history.  Capacity = throughput with every
    request queued at once; then Poisson arrivals at 50% and 80% of it.  With
    a host tier attached, evicted users are offloaded and onboarded instead."""
    from generative_recommender_sequence_amd import serving

    cfg = w.cfg
    out = {"users": users, "max_batch": 8, "max_delay_us": 500, "in_flight": 2}
    for label, host in (("device_cache", False), ("with_host_tier", True)):
        rng = np.random.default_rng([seed, 77])
        pop = serving.Population.draw(rng, users, cfg, events=(0, 16))
        longest = pop.max_hist + 16 + cfg.n_targets
        max_pages = -(-longest // cfg.page_size)
        half = sum(-(-(int(h) + 16 + cfg.n_targets) // cfg.page_size) for h in pop.hist) // 2
        pages = max(half, 8 * max_pages)
        host_pages = 2 * users * max_pages if host else 0
        srv = serving.Server(cfg, w.layers, pop, pages, host_pages=host_pages, seed=seed)
        srv.run(serving.poisson_arrivals(rng, pop, float("inf"), 160))            # warm the cache
        cap = srv.run(serving.poisson_arrivals(rng, pop, float("inf"), 800)).summary()
        res = {"pool_pages": pages, "host_pages": host_pages, "capacity": cap}
        for frac in (0.5, 0.8):
            rate = frac * cap["throughput_req_per_s"]
            res[f"load_{int(frac * 100)}pct"] = dict(
                offered_req_per_s=round(rate, 1),
                **srv.run(serving.poisson_arrivals(rng, pop, rate, 1200)).summary())
        out[label] = res
        del srv
    return out


def scn_evicted(scn, users, new_len):
    from generative_recommender_sequence_amd import hstu
    if scn.cache is None:
        return []
    scn.restore()
    cached = hstu.kv_lookup(scn.cache.h, users)
    need = scn.cache.pages_needed(cached, new_len)
    ev = hstu.kv_evict_lru(scn.cache.h, need, users) if hstu.kv_free_pages(scn.cache.h) < need else []
    scn.restore()
    return ev


def cpu_baseline(w, scn, users, new_len, n_targets, norm_n, rows):
    """The oracle on layer 0 of the same request (every user; hit users attend
    to a seeded random history of their cached length), scaled to the stack's
    layer count."""
    import oracle

    cfg = w.cfg
    inner = cfg.inner
    cached = [int(w.hist_len[b]) if w.hit[b] else 0 for b in range(cfg.batch)]
    rng = np.random.default_rng(1234)
    hk = rng.standard_normal((sum(cached), inner)) * 0.1
    hv = rng.standard_normal((sum(cached), inner)) * 0.1
    x = np.concatenate(rows).astype(np.float64)
    t0 = time.perf_counter()
    oracle.layer(x, w.layers[0].w1, w.layers[0].w2, w.layers[0].rab, new_len, cached, n_targets, norm_n, hk, hv,
                 cfg.num_heads, cfg.head_dim, cfg.eps)
    dt = time.perf_counter() - t0
    per_step = dt * cfg.num_layers
    return {"value": round(sum(new_len) / per_step, 2), "unit": "new tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"layer 0 of one {cfg.name} request ({sum(new_len)} new tokens, all {cfg.batch} users), "
                      f"{dt:.1f} s, scaled by {cfg.num_layers} layers"}


if __name__ == "__main__":
    main()

"""Benchmark of the HSTU block forward with a paged KV cache on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C4]

One step is one whole request through the hot path: restore the cache
metadata to its pre-request state, look the batch up, evict least-recently
used users if pages are short, allocate pages, upload the page table and the
request plan, then run every layer (pre-norm, f1 + SiLU, K/V append,
attention over cached + new keys, LayerNorm(AV) * U, f2 + residual) on the
new tokens, and score the candidate rows with the multitask ranking head.
The new-token inputs are already in device memory when timing starts.

Prints one JSON line: new tokens per second of the headline workload, its
dominant kernel against its roofline (duration from HIP events on its launch
stream), the attention of users with and without a cached prefix timed as
separate launches, request latency percentiles, the other cached workloads
(C3, C5) with their attention against the HBM roofline, measured achievable
ceilings beside the vendor peaks, and the CPU oracle timed on a bounded
sample of the same workload.
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


def user_pairs(c: int, t: int, T: int) -> int:
    """Unmasked (query, key) pairs per head of one user's new queries c..c+t-1
    (history queries see j <= i, the last T positions see the history and
    themselves)."""
    L = c + t
    hist = L - T
    pairs = 0
    if c < hist:
        pairs += (hist * (hist + 1) - c * (c + 1)) // 2
    pairs += max(0, L - max(c, hist)) * (hist + 1)
    return pairs


def attention_bytes(cached_len, new_len, H, dh, es=2):
    """Algorithmic HBM bytes of attention over these users: every key/value
    row of a user with new tokens once per head, the queries once, the fp32
    output once."""
    kv = sum(int(c + t) for c, t in zip(cached_len, new_len) if t > 0)
    n = int(sum(new_len))
    return kv * H * dh * 2 * es + n * H * dh * (es + 4)


def attention_flops(cached_len, new_len, n_targets, H, dh):
    """4 dh FLOPs per unmasked pair and head (q.k and the weighted sum of v)."""
    return 4.0 * dh * H * sum(user_pairs(int(c), int(t), int(T)) for c, t, T in zip(cached_len, new_len, n_targets))


def hbm_roof(nbytes, us, ceil):
    achieved = nbytes / (us * 1e-6) / 1e9
    out = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "frac": round(achieved / PEAK_HBM_GBS, 4)}
    if ceil:
        out.update(achievable_peak=round(ceil, 1), frac_of_achievable=round(achieved / ceil, 4))
    return out


def mfma_roof(flops, us, ceil):
    achieved = flops / (us * 1e-6) / 1e12
    out = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
           "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    if ceil:
        out.update(achievable_peak=round(ceil, 1), frac_of_achievable=round(achieved / ceil, 4))
    return out


def ceilings():
    """Achievable peaks measured on this GPU with the library's ceiling
    kernels (bf16 MFMA issue rate, streaming read, copy), each the best of 5
    event-timed launches."""
    import torch

    from generative_recommender_sequence_amd import hstu, runtime
    s = runtime.stream_handle()
    out = torch.zeros(1 << 16, dtype=torch.float32, device="cuda")

    def best(fn, reps=5):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    blocks, iters = 256 * 8, 2048
    ms = best(lambda: hstu.hstu_ceiling_mfma(blocks, iters, out.data_ptr(), s))
    mfma = blocks * 4 * 4 * iters * 32768 / (ms * 1e-3) / 1e12
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    ms = best(lambda: hstu.hstu_ceiling_read(buf.data_ptr(), nbytes, out.data_ptr(), s))
    read = nbytes / (ms * 1e-3) / 1e9
    half = nbytes // 2
    ms = best(lambda: hstu.hstu_ceiling_copy(buf.data_ptr(), buf.data_ptr() + half, half, s))
    copy = 2 * half / (ms * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma, 1), "hbm_read_GBps": round(read, 1),
            "hbm_copy_GBps_read_plus_write": round(copy, 1),
            "method": "library ceiling kernels (hstu_ceiling_*): 2048 blocks x 4 waves x 8192 back-to-back "
                      "32x32x16 bf16 MFMAs; a 4 GiB streaming read; a 2 GiB copy; best of 5 event-timed launches"}


class Run:
    """One workload's request loop on the GPU."""

    def __init__(self, w, seed, head=True):
        import torch

        from generative_recommender_sequence_amd import runtime
        from generative_recommender_sequence_amd.workloads import head_weights
        self.w, self.cfg = w, w.cfg
        cfg = self.cfg
        self.scn = scn = runtime.Scenario(w)
        scn.prefill()
        self.users, self.new_len, self.n_targets, self.norm_n, rows = scn.request_inputs()
        self.rows = rows
        self.x = scn._x(rows)                        # new-token inputs resident in HBM
        self.n_new = int(sum(self.new_len))
        scn.restore()
        req0 = scn.make_request(rows)[0]
        self.ws = runtime.workspace_for(scn.model, req0)
        self.info0 = req0.info
        self.cached_len = np.asarray(req0.cached_len)
        req0.close()
        self.rbufs = runtime.RequestBuffers(cfg.batch, scn.max_pages, int(self.info0.meta_bytes) + 4096)
        self.ybufs = [torch.empty_like(self.x), torch.empty_like(self.x)]
        self.head = runtime.Head(head_weights(cfg.d_model, seed=seed), scn.dtype) if head else None
        self.cand = torch.from_numpy(runtime.candidate_row_list(self.new_len, self.n_targets)).cuda()
        self.logits = torch.empty((max(self.cand.numel(), 1), 4), dtype=torch.float32, device="cuda")

    def step(self):
        from generative_recommender_sequence_amd import runtime
        scn, cfg = self.scn, self.cfg
        scn.restore()
        req = runtime.prepare(scn.cache, self.users, self.new_len, self.n_targets, self.norm_n, scn.max_pages,
                              cfg.num_heads, cfg.head_dim, bufs=self.rbufs)
        y = runtime.forward(scn.model, req, self.x, scn.cache, self.ws, out_bufs=self.ybufs)
        if self.head is not None:
            self.head(y, self.cand, out=self.logits)
        return req

    def loop(self, steps):
        """steps back-to-back requests (host work of request k+1 overlaps the
        GPU work of request k); returns ms per request."""
        import torch
        pending = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            pending.append(self.step())
        torch.cuda.synchronize()
        ms = 1000.0 * (time.perf_counter() - t0) / steps
        for r in pending:
            r.close()
        return ms

    def warmup(self, n, min_s=0.3):
        import torch
        t0, k, pending = time.perf_counter(), 0, []
        while k < n or time.perf_counter() - t0 < min_s:
            pending.append(self.step())
            k += 1
            if len(pending) >= 16:
                torch.cuda.synchronize()
                for r in pending:
                    r.close()
                pending.clear()
        torch.cuda.synchronize()
        for r in pending:
            r.close()
        return k

    def latency(self, n):
        """Per-request latency: each request alone on an idle GPU, from an
        event recorded before its host work (cache operations, plan, uploads)
        to one recorded after its last kernel; p50 / p90 over n requests."""
        import torch
        lat = []
        for _ in range(n):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            req = self.step()
            e1.record()
            e1.synchronize()
            lat.append(e0.elapsed_time(e1))
            req.close()
        a = np.asarray(lat)
        return {"p50": round(float(np.percentile(a, 50)), 4), "p90": round(float(np.percentile(a, 90)), 4),
                "mean": round(float(a.mean()), 4), "requests": n}

    def kernels(self, steps, split=False):
        """The same requests with every kernel bracketed by HIP events on its
        launch stream; split: the attention of users with and without a cached
        prefix as two launches."""
        import torch

        from generative_recommender_sequence_amd import hstu
        hstu.hstu_timing_enable(True, split_attention=split)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ms = self.loop(steps)
        del t0
        kern = {}
        for name in hstu.TIMED_KERNELS:
            n, tot = hstu.hstu_timing_read(name)
            if n:
                kern[name] = {"launches": n, "avg_us": round(1000.0 * tot / n, 2),
                              "ms_per_step": round(tot / steps, 4)}
        hstu.hstu_timing_enable(False)
        return kern, ms


    def phases(self, steps=3):
        """Per-block phase records of the attention launch (the last layer of
        the last of `steps` requests): set-up, key-tile loop and partial-tile
        write times, the launch span, the share of the span the chip's block
        slots were busy, and when each XCD ran out of work."""
        import torch

        from generative_recommender_sequence_amd import hstu
        n = int(self.info0.n_work_items)
        rec = hstu.ATTN_STAMP_DTYPE.itemsize
        buf = torch.zeros(n * rec // 8 + 8, dtype=torch.int64, device="cuda")
        hstu.hstu_attn_stamps(buf.data_ptr(), n)
        try:
            self.loop(steps)
        finally:
            torch.cuda.synchronize()
            hstu.hstu_attn_stamps(0, 0)
        a = np.frombuffer(buf.cpu().numpy().tobytes()[:n * rec], dtype=hstu.ATTN_STAMP_DTYPE)
        return summarize_phases(a)


def summarize_phases(a):
    """Summary of one attention launch's phase records (hstu_attn_stamps):
    set-up, per-tile loop and write times (p10/p50/p90/max over blocks), the
    launch span, the CUs used, when each XCD and each CU ran out of work, and
    the share of the span the CUs' two block slots were busy."""
    a = a[a["end"] > 0]
    if len(a) == 0:
        return None
    ns = 10.0  # the realtime counter runs at 100 MHz
    t0 = int(a["start"].min())
    span = (int(a["end"].max()) - t0) * ns / 1000.0
    setup = (a["setup_done"] - a["start"]) * ns / 1000.0
    loop = (a["loop_done"] - a["setup_done"]) * ns / 1000.0
    write = (a["end"] - a["loop_done"]) * ns / 1000.0
    tiles = np.maximum(a["tiles"], 1)
    cu = a["xcc_id"].astype(np.int64) * 256 + ((a["hw_id"] >> 8) & 0xFF)
    n_cu = len(np.unique(cu))
    busy = float(((a["end"] - a["start"]) * ns / 1000.0).sum())
    xcd_end = {int(x): round((int(a["end"][a["xcc_id"] == x].max()) - t0) * ns / 1000.0, 2)
               for x in np.unique(a["xcc_id"])}
    cu_end = np.array([(int(a["end"][cu == c].max()) - t0) * ns / 1000.0 for c in np.unique(cu)])

    def q(v):
        return {"p10": round(float(np.percentile(v, 10)), 3), "p50": round(float(np.percentile(v, 50)), 3),
                "p90": round(float(np.percentile(v, 90)), 3), "max": round(float(v.max()), 3)}
    return {"blocks": int(len(a)), "cus_used": n_cu, "span_us": round(span, 2),
            "setup_us": q(setup), "tile_loop_us_per_tile": q(loop / tiles), "tiles_per_block": q(a["tiles"]),
            "write_us": q(write),
            "busy_share": round(busy / (2 * max(n_cu, 1) * span), 3) if span > 0 else None,
            "xcd_last_end_us": xcd_end,
            "cu_last_end_us": q(cu_end),
            "note": ("realtime-clock stamps (10 ns) written by every attention block of one launch (the last "
                     "layer of a request); busy_share = summed block time / (2 resident blocks x CUs used x "
                     "span)")}


def measure(name, seed, steps, warmup, latency_n, ceil, split=False):
    """ms per request, latency, per-kernel times and the attention roofline of
    one workload."""
    from generative_recommender_sequence_amd import profiling
    from generative_recommender_sequence_amd.workloads import workload_for
    w = workload_for(name, seed)
    run = Run(w, seed)
    cfg = run.cfg
    H, dh = cfg.num_heads, cfg.head_dim
    n_w = run.warmup(warmup)
    ms = run.loop(steps)
    kern, ms_instr = run.kernels(steps)
    lat = run.latency(latency_n)
    cached, new, T = run.cached_len, np.asarray(run.new_len), np.asarray(run.n_targets)
    att_us = kern["attention"]["avg_us"]
    flops = attention_flops(cached, new, T, H, dh)
    nbytes = attention_bytes(cached, new, H, dh)
    if cfg.cache == "hit":
        roof = hbm_roof(nbytes, att_us, ceil and ceil["hbm_read_GBps"])
    else:
        roof = mfma_roof(flops, att_us, ceil and ceil["mfma_bf16_tflops"])
    traffic = profiling.read_traffic(name)
    roof["traffic"] = None if traffic is None else round(traffic, 0)
    roof.update({"kernel": "attention (attn_bf16_kernel, paged)", "avg_us": att_us,
                 "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes,
                 "unmasked_pairs_per_head": int(flops / (4 * dh * H))})
    res = {"workload": f"{name}: {WORKLOAD_TEXT[name]}", "new_tokens_per_step": run.n_new,
           "candidate_tokens_per_step": int(T.sum()), "ms_per_step": round(ms, 4),
           "new_tokens_per_s": round(run.n_new / (ms / 1000.0), 1),
           "ms_per_step_event_instrumented": round(ms_instr, 4), "warmup_steps_run": n_w,
           "latency_ms": lat, "roofline": roof, "kernels": kern,
           "kernel_ms_per_step": round(sum(k["ms_per_step"] for k in kern.values()), 4),
           "attention_work_items": int(run.info0.n_work_items)}
    res["attention_phases"] = run.phases()
    if split:
        ks, _ = run.kernels(steps, split=True)
        hit = cached > 0
        out = {}
        if "attention_cached" in ks:
            nb = attention_bytes(cached[hit], new[hit], H, dh)
            fl = attention_flops(cached[hit], new[hit], T[hit], H, dh)
            us = ks["attention_cached"]["avg_us"]
            out["cached_prefix_users"] = dict(users=int(hit.sum()), avg_us=us, algorithmic_bytes=nb,
                                              algorithmic_flops=fl,
                                              **hbm_roof(nb, us, ceil and ceil["hbm_read_GBps"]))
        if "attention_prefill" in ks:
            fl = attention_flops(cached[~hit], new[~hit], T[~hit], H, dh)
            us = ks["attention_prefill"]["avg_us"]
            out["full_recompute_users"] = dict(users=int((~hit).sum()), avg_us=us, algorithmic_flops=fl,
                                               **mfma_roof(fl, us, ceil and ceil["mfma_bf16_tflops"]))
        out["note"] = ("same requests, instrumented pass whose attention runs the users with a cached prefix "
                       "and the users without one as two grids; the headline pass runs them as one grid")
        res["attention_split"] = out
    res["_run"] = run
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="C4", choices=["C2", "C3", "C4", "C5"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--latency-requests", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-serving", action="store_true", help="skip the serving-loop latency measurement")
    ap.add_argument("--no-training", action="store_true", help="skip the training-step measurement")
    ap.add_argument("--no-extra", action="store_true",
                    help="headline workload only: no cached-path workloads, ceilings, 8-layer context, "
                         "host tier, serving or training")
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
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 (a request's users are "
                                   "independent, so more GPUs would each serve their own users)"}), flush=True)
        sys.exit(2)

    import torch

    from generative_recommender_sequence_amd import runtime

    runtime.require_gpu()
    torch.cuda.set_device(0)
    extra = not args.no_extra
    ceil = ceilings() if extra else None
    main_res = measure(args.workload, args.seed, args.steps, args.warmup, args.latency_requests, ceil,
                       split=args.workload == "C4")
    run = main_res.pop("_run")
    w, cfg, scn = run.w, run.cfg, run.scn
    users, new_len, n_targets, norm_n, rows = run.users, run.new_len, run.n_targets, run.norm_n, run.rows
    n_evicted = int(len(scn_evicted(scn, users, new_len)))
    tier = host_tier_rates(scn) if (extra and scn.cache is not None) else None   # attaches a host tier
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, users, new_len, n_targets, norm_n, rows)
    del run, scn
    torch.cuda.empty_cache()

    cached_path = None
    if extra:
        cached_path = {}
        for name in ("C3", "C5"):
            if name == args.workload:
                continue
            r = measure(name, args.seed, max(5, args.steps // 2), 3, max(10, args.latency_requests // 3), ceil)
            r.pop("_run")
            cached_path[name] = r
            torch.cuda.empty_cache()
    context = c3_eight_layers(args.seed) if extra else None
    serving_out = None
    if extra and not args.no_serving and args.workload == "C4":
        serving_out = serving_results(w, args.seed)
    training_out = None
    if extra and not args.no_training and args.workload == "C4":
        training_out = training_results(args.seed, ceil)

    ms_per_step = main_res["ms_per_step"]
    roof = main_res["roofline"]
    out = {
        "metric": "HSTU new tokens/s at batch 8, 8 layers, cache hit; % HBM / MFMA roofline",
        "value": main_res["new_tokens_per_s"],
        "unit": "new tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": main_res["warmup_steps_run"],
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal weights/inputs, random-init; shapes of the pages' benchmark)",
        "config": {"workload": main_res["workload"], "global_batch": cfg.batch,
                   "layers": cfg.num_layers, "d_model": cfg.d_model, "heads": cfg.num_heads,
                   "head_dim": cfg.head_dim,
                   "new_tokens_per_step": main_res["new_tokens_per_step"],
                   "candidate_tokens_per_step": main_res["candidate_tokens_per_step"],
                   "cached_key_fraction": round(float(run_cached_fraction(w)), 4),
                   "evicted_users_per_step": n_evicted,
                   "attention_work_items": main_res["attention_work_items"],
                   "head": "4 tasks x MLP(512-256-1) on every candidate row",
                   "seed": args.seed},
        "roofline": roof,
        "attention_split": main_res.get("attention_split"),
        "attention_phases": main_res.get("attention_phases"),
        "latency_ms": main_res["latency_ms"],
        "kernels": main_res["kernels"],
        "kernel_ms_per_step": main_res["kernel_ms_per_step"],
        "ms_per_step_event_instrumented": main_res["ms_per_step_event_instrumented"],
        "candidate_tokens_per_s": round(main_res["candidate_tokens_per_step"] / (ms_per_step / 1000.0), 1),
        "ceilings": ceil,
        "cached_path": cached_path,
        "c3_setup_at_8_layers": context,
        "host_tier": tier,
        "serving": serving_out,
        "training": training_out,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def run_cached_fraction(w):
    cached = sum(int(w.hist_len[b]) for b in range(w.cfg.batch) if w.hit[b])
    total = sum(int(w.hist_len[b] + w.n_targets[b]) for b in range(w.cfg.batch))
    return cached / max(total, 1)


def c3_eight_layers(seed, steps=10):
    """Context only, not scored: C3's setup (batch 8, histories uniform [1024,
    4096], 64 candidates, 32-token pages, 100% hit) at 8 layers, against the
    same 8-layer stack recomputing every user's history (no cache); the
    pages quote their cache-vs-no-cache latency ratio for an 8-layer model
    at batch 8 with every history cached."""
    import dataclasses

    import torch

    from generative_recommender_sequence_amd.workloads import workload_for
    w = workload_for("C3", seed, num_layers=8)
    out = {}
    for label, ww in (("cached", w), ("no_cache", dataclasses.replace(
            w, cfg=dataclasses.replace(w.cfg, cache="none"), hit=np.zeros(w.cfg.batch, bool)))):
        run = Run(ww, seed)
        run.warmup(3)
        ms = run.loop(steps)
        lat = run.latency(10)
        out[label] = {"ms_per_request": round(ms, 4), "latency_ms_p50": lat["p50"],
                      "new_tokens_per_request": run.n_new}
        del run
        torch.cuda.empty_cache()
    out["latency_ratio_no_cache_over_cached"] = round(out["no_cache"]["latency_ms_p50"] /
                                                      out["cached"]["latency_ms_p50"], 2)
    out["note"] = ("context only: the pages' 8-layer figure is a latency ratio measured on other hardware and "
                   "another serving stack")
    return out


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


def training_results(seed, ceil, steps=5, warmup=2):
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
    roof = mfma_roof(flops, bwd_att_ms * 1000.0, ceil and ceil["mfma_bf16_tflops"])
    roof.update(algorithmic_flops_per_layer=flops, ms_per_layer=round(bwd_att_ms, 4))
    req.close()
    return {"workload": "C2 model and batch: 3 bf16 layers, batch 8, histories uniform [1024, 4096] + 64 "
                        "candidates, forward (with taps) + backward, seeded dL/dY",
            "tokens_per_step": n, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(n / (ms / 1000.0), 1),
            "kernels_ms_per_step": {k: v["ms_per_step"] for k, v in kern.items()},
            "backward_attention_roofline": roof}


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


def cpu_baseline(w, users, new_len, n_targets, norm_n, rows):
    """The oracle on layer 0 of the same request (every user; hit users attend
    to a seeded random history of their cached length), scaled to the stack's
    layer count, with all host threads; then single-threaded on a smaller
    sample (the cached users and the two shortest recomputed ones), beside the
    all-threads time of that sample."""
    import oracle

    cfg = w.cfg
    inner = cfg.inner
    cached = [int(w.hist_len[b]) if w.hit[b] else 0 for b in range(cfg.batch)]
    rng = np.random.default_rng(1234)

    def run(sel):
        c = [cached[b] for b in sel]
        hk = rng.standard_normal((sum(c), inner)) * 0.1
        hv = rng.standard_normal((sum(c), inner)) * 0.1
        x = np.concatenate([rows[b] for b in sel]).astype(np.float64)
        t0 = time.perf_counter()
        oracle.layer(x, w.layers[0].w1, w.layers[0].w2, w.layers[0].rab, [new_len[b] for b in sel], c,
                     [n_targets[b] for b in sel], [norm_n[b] for b in sel], hk, hv, cfg.num_heads, cfg.head_dim,
                     cfg.eps)
        return time.perf_counter() - t0, int(sum(new_len[b] for b in sel))

    threads = oracle.threads()
    dt, toks = run(list(range(cfg.batch)))
    out = {"value": round(toks / (dt * cfg.num_layers), 2), "unit": "new tokens/s", "cores": threads,
           "kind": "oracle",
           "sample": f"layer 0 of one {cfg.name} request ({toks} new tokens, all {cfg.batch} users), "
                     f"{dt:.1f} s, scaled by {cfg.num_layers} layers"}
    L = [int(w.hist_len[b] + w.n_targets[b]) for b in range(cfg.batch)]
    miss = sorted((b for b in range(cfg.batch) if not cached[b]), key=lambda b: L[b])
    sel = sorted([b for b in range(cfg.batch) if cached[b]] + miss[:2])
    dt_all, toks_s = run(sel)
    oracle.set_threads(1)
    try:
        dt_one, _ = run(sel)
    finally:
        oracle.set_threads(threads)
    out["single_thread"] = {
        "value": round(toks_s / (dt_one * cfg.num_layers), 2), "unit": "new tokens/s", "cores": 1,
        "sample": f"layer 0 of users {sel} of the same request ({toks_s} new tokens: the cached users and the "
                  f"two shortest recomputed ones), {dt_one:.1f} s, scaled by {cfg.num_layers} layers",
        "same_sample_all_threads": round(toks_s / (dt_all * cfg.num_layers), 2)}
    return out


if __name__ == "__main__":
    main()

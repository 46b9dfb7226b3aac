"""A serving loop over the library: dynamic batching of a stream of user
requests, with host-side cache operations overlapped with the GPU work of the
batch before.

The pages serve the HSTU ranking model through Dynamo-Triton at dynamic batch
size 8 with a KV cache ("NVIDIA Dynamo-Triton Gets End-to-End HSTU Generative
Recommender Workflow", section Five stages and the benchmark; "Deploying an
HSTU Generative Recommender with NVIDIA Dynamo-Triton", KV cache section).
Here a request is one user: the history events that arrived since the user's
last request plus T candidates to score.  A batch of requests:

  host  residency -> the user's cached length c_u (0 on a miss; a user found
        on the host tier is onboarded), new tokens = (history h_u - c_u) + T,
        lookup / LRU eviction (or offload) / allocation, page table and plan
        upload (runtime.prepare);
  GPU   the layer stack on the new tokens, the multitask head on the
        candidate rows, logits copied to pinned host memory;
  host  each user's cache is cut back to its history (the candidates are
        scored, not remembered).

Every device step of every batch goes on one stream, so the host may prepare
batch k+1 (and evict, reuse or cut pages) while batch k still runs: the GPU
work that reads a page is ordered before the work that overwrites it.  At
most `depth` batches are in flight.
"""
from __future__ import annotations

import time
from collections import deque
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import hstu, runtime
from .workloads import HEAD_HIDDEN, HEAD_TASKS, Config, head_weights, round_bf16


@dataclass
class Population:
    """Users with a persistent history that grows between their requests."""
    hist: np.ndarray          # [U] current history length h_u
    events: tuple             # new history events per request: uniform [lo, hi]
    n_targets: int
    max_hist: int

    @classmethod
    def draw(cls, rng, n_users: int, cfg: Config, events=(0, 16)) -> "Population":
        kind, med, lo, hi = cfg.hist
        assert kind == "lognormal"
        h = np.clip(np.rint(med * np.exp(rng.standard_normal(n_users))), lo, hi).astype(np.int64)
        return cls(h, events, cfg.n_targets, hi)


@dataclass
class Arrival:
    t: float      # seconds after the start
    user: int
    events: int   # history events that came with the request


def poisson_arrivals(rng, pop: Population, rate: float, n: int, t0: float = 0.0) -> List[Arrival]:
    """n requests, exponential gaps at `rate` per second (rate = inf: all at
    t0), users uniform over the population."""
    gaps = np.zeros(n) if not np.isfinite(rate) else rng.exponential(1.0 / rate, size=n)
    ts = t0 + np.cumsum(gaps)
    users = rng.integers(0, len(pop.hist), size=n)
    ev = rng.integers(pop.events[0], pop.events[1] + 1, size=n)
    return [Arrival(float(t), int(u), int(e)) for t, u, e in zip(ts, users, ev)]


@dataclass
class ServeStats:
    latencies_ms: List[float] = field(default_factory=list)
    batch_sizes: List[int] = field(default_factory=list)
    hits: int = 0
    onboarded: int = 0
    tokens: int = 0
    elapsed_s: float = 0.0

    def summary(self) -> dict:
        lat = np.asarray(self.latencies_ms)
        n = len(lat)
        return {"requests": n,
                "throughput_req_per_s": round(n / self.elapsed_s, 1) if self.elapsed_s else None,
                "new_tokens_per_s": round(self.tokens / self.elapsed_s, 1) if self.elapsed_s else None,
                "latency_ms_p50": round(float(np.percentile(lat, 50)), 3) if n else None,
                "latency_ms_p90": round(float(np.percentile(lat, 90)), 3) if n else None,
                "latency_ms_p99": round(float(np.percentile(lat, 99)), 3) if n else None,
                "latency_ms_mean": round(float(lat.mean()), 3) if n else None,
                "mean_batch": round(float(np.mean(self.batch_sizes)), 2) if self.batch_sizes else None,
                "hit_rate": round(self.hits / n, 3) if n else None,
                "onboarded": self.onboarded}


class Server:
    """The model, head, cache and the buffers a stream of batches reuses."""

    def __init__(self, cfg: Config, layers, pop: Population, num_pages: int, host_pages: int = 0,
                 max_batch: int = 8, max_delay_us: int = 500, depth: int = 2, seed: int = 0,
                 device="cuda"):
        self.cfg, self.pop, self.depth, self.device = cfg, pop, depth, device
        self.dtype = runtime.dtype_code(cfg.dtype)
        self.model = runtime.Model(layers, self.dtype, cfg.num_heads, cfg.head_dim, cfg.d_model, cfg.eps, device)
        self.head = runtime.Head(head_weights(cfg.d_model, HEAD_TASKS, HEAD_HIDDEN, seed, cfg.dtype), self.dtype,
                                 device)
        self.cache = runtime.PagedCache(cfg.num_layers, cfg.num_heads, cfg.head_dim, cfg.page_size, num_pages,
                                        self.dtype, None, device, zero=False)
        if host_pages:
            self.cache.attach_host(host_pages)
        longest = pop.max_hist + pop.events[1] + pop.n_targets
        self.max_pages = -(-longest // cfg.page_size)
        if num_pages < max_batch * self.max_pages:
            raise ValueError(f"a pool of {num_pages} pages cannot hold a batch of {max_batch} users of up to "
                             f"{self.max_pages} pages")
        self.max_rows = max_batch * longest
        rng = np.random.default_rng([seed, 0x5E5])
        x = round_bf16(rng.standard_normal((self.max_rows, cfg.d_model)).astype(np.float32))
        self.x = torch.from_numpy(x).to(device=device, dtype=runtime.tdtype(self.dtype))
        self.ybufs = [torch.empty_like(self.x), torch.empty_like(self.x)]
        self.bufs = runtime.RequestBuffers(max_batch, self.max_pages, 1 << 20, device, slots=depth + 1)
        # per in-flight slot: candidate rows (pinned -> device) and logits (device -> pinned);
        # a slot is reused only after the batch that last used it has been retired
        rows = max_batch * pop.n_targets
        slots = depth + 1
        self.rows_host = [torch.empty(rows, dtype=torch.int32, pin_memory=True) for _ in range(slots)]
        self.rows_dev = [torch.empty(rows, dtype=torch.int32, device=device) for _ in range(slots)]
        self.logits_dev = [torch.empty((rows, HEAD_TASKS), dtype=torch.float32, device=device)
                           for _ in range(slots)]
        self.logits_host = [torch.empty((rows, HEAD_TASKS), dtype=torch.float32, pin_memory=True)
                            for _ in range(slots)]
        self.slot = 0
        self.batcher = hstu.Batcher(max_batch, max_delay_us, 0)
        # observer of each launch: (request ids, users, cached lengths, histories, new lengths)
        self.on_launch = None

    def launch(self, ids: List[int], arrivals: List[Arrival], stats: ServeStats):
        """Host cache ops and the batch's GPU work; returns (event, slot)."""
        cfg, pop, cache = self.cfg, self.pop, self.cache
        users = np.array([a.user for a in arrivals], np.int64)
        for a in arrivals:
            pop.hist[a.user] = min(pop.hist[a.user] + a.events, pop.max_hist + pop.events[1])
        where, cached = hstu.kv_residency(cache.h, users)
        hist = pop.hist[users]
        new_len = (hist - np.minimum(cached, hist) + pop.n_targets).astype(np.int32)
        n_targets = np.full(len(users), pop.n_targets, np.int32)
        norm_n = (hist + pop.n_targets).astype(np.float32)
        req = runtime.prepare(cache, users, new_len, n_targets, norm_n, self.max_pages, cfg.num_heads,
                              cfg.head_dim, self.device, bufs=self.bufs)
        if self.on_launch is not None:
            self.on_launch(list(ids), users.copy(), req.cached_len.copy(), hist.copy(), new_len.copy())
        stats.hits += int(np.count_nonzero(req.cached_len))
        stats.onboarded += len(req.onboarded)
        n_new = int(new_len.sum())
        stats.tokens += n_new
        x = self.x[:n_new]
        ws = runtime.workspace_for(self.model, req, self.device)
        y = runtime.forward(self.model, req, x, cache, ws, out_bufs=self.ybufs)
        cand = runtime.candidate_row_list(new_len, n_targets)
        n_cand = len(cand)
        k = self.slot
        self.slot = (self.slot + 1) % len(self.logits_dev)
        self.rows_host[k].numpy()[:n_cand] = cand
        self.rows_dev[k][:n_cand].copy_(self.rows_host[k][:n_cand], non_blocking=True)
        self.head(y, self.rows_dev[k], n_cand, out=self.logits_dev[k])
        self.logits_host[k][:n_cand].copy_(self.logits_dev[k][:n_cand], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        # the candidates are scored, not remembered: cut each user back to its history
        for u, h in zip(users, hist):
            hstu.kv_truncate(cache.h, int(u), int(h))
        req.close()
        return ev, k

    def run(self, arrivals: List[Arrival], keep_logits: Optional[dict] = None) -> ServeStats:
        """Serves `arrivals` in real time; latency = completion seen by the
        host - arrival.  keep_logits (a dict): request index -> its [T, tasks]
        logits."""
        stats = ServeStats()
        pending = {}
        inflight = deque()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        i, done, n = 0, 0, len(arrivals)
        while done < n:
            now = time.perf_counter() - t0
            while i < n and arrivals[i].t <= now:
                a = arrivals[i]
                self.batcher.submit(i, a.user, 0, int(a.t * 1e6))
                pending[i] = a
                i += 1
            while inflight and inflight[0][0].query():
                _, k, ids = inflight.popleft()
                t_done = time.perf_counter() - t0
                for j, rid in enumerate(ids):
                    stats.latencies_ms.append(1000.0 * (t_done - arrivals[rid].t))
                    if keep_logits is not None:
                        T = self.pop.n_targets
                        keep_logits[rid] = self.logits_host[k][j * T:(j + 1) * T].numpy().copy()
                done += len(ids)
            if len(inflight) < self.depth:
                ids, wait = self.batcher.next(int(now * 1e6))
                if ids:
                    ev, k = self.launch(ids, [pending.pop(r) for r in ids], stats)
                    inflight.append((ev, k, ids))
                    stats.batch_sizes.append(len(ids))
                    continue
            time.sleep(0)
        stats.elapsed_s = time.perf_counter() - t0
        return stats

"""Seeded synthetic workloads for the HSTU block forward.

This module only draws numbers: lengths, user ids, weights, relative-bias
tables, input embeddings and the physical page permutation.  It holds none of
the method's arithmetic, so both the HIP path and the CPU oracle can consume
its output.  The shapes follow the workloads described on the pages
("Deploying an HSTU Generative Recommender with NVIDIA Dynamo-Triton",
benchmark details: hidden size 512, 4 attention heads, BF16 weights, 3- and
8-layer models, batch 8, histories up to 8192 tokens); the KuaiRand-1K data
those pages measure on is not available, and seeded normal draws of the same
shapes stand in for it.

Draw order (numpy PCG64, one generator per workload):
  1. history lengths of the batch users
  2. (mixed cache only) the hit mask, then the stale users' history lengths
  3. user ids (a permutation, so batch order differs from id order)
  4. the order in which cached users were pre-filled (their prior LRU ticks)
  5. per layer: W1, W2, rab
  6. X: per batch user history then candidates, then per stale user history
  7. the physical page permutation of the pool
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import List, Optional

import numpy as np


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern (uint16) -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16, returned as float32."""
    return bf16_to_f32(bf16_bits(a))


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str                 # "f32" or "bf16"
    batch: int
    d_model: int
    num_heads: int
    head_dim: int
    num_layers: int
    hist: tuple                # ("fixed", (l0, l1, ...)) | ("uniform", lo, hi) | ("lognormal", median, lo, hi)
    n_targets: int             # candidate tokens per user (0 = pure causal)
    cache: str                 # "none" | "hit" | "mixed"
    page_size: int = 32
    num_buckets: int = 64
    eps: float = 1e-5
    hit_fraction: float = 0.5  # mixed cache only
    n_stale: int = 0           # mixed cache only: users cached before the request, not in it
    seed_alias: Optional[str] = None  # draw the data of another workload (same seed)

    @property
    def inner(self) -> int:
        return self.num_heads * self.head_dim


CONFIGS = {
    # tiny single layer, fp32, causal, no cache
    "C1": Config("C1", "f32", 2, 64, 2, 32, 1, ("fixed", (37, 64)), 0, "none"),
    # 3-layer bf16 stack, full recompute, 64 target-aware candidates per user
    "C2": Config("C2", "bf16", 8, 512, 4, 128, 3, ("uniform", 1024, 4096), 64, "none"),
    # the same model and histories with every user's history cached in 32-token pages
    "C3": Config("C3", "bf16", 8, 512, 4, 128, 3, ("uniform", 1024, 4096), 64, "hit",
                 page_size=32, seed_alias="C2"),
    # 8-layer stack, half the users hit, the rest prefill; pool forces LRU eviction
    "C4": Config("C4", "bf16", 8, 512, 4, 128, 8, ("lognormal", 2048, 256, 8192), 64, "mixed",
                 page_size=32, hit_fraction=0.5, n_stale=8),
    # throughput stress: batch 128, 256 candidates, 64-token pages, 128 buckets
    "C5": Config("C5", "bf16", 128, 512, 4, 128, 8, ("lognormal", 2048, 128, 16384), 256, "hit",
                 page_size=64, num_buckets=128),
}


@dataclass
class LayerWeights:
    w1: np.ndarray   # [d, 4*H*dh] float32 (bf16-exact in bf16 workloads); columns [U|V|Q|K], head-major
    w2: np.ndarray   # [H*dh, d]
    rab: np.ndarray  # [num_buckets]


@dataclass
class HeadWeights:
    """Multitask ranking head, per task t: a [t] [d][hidden] first-layer
    weights (bf16-exact in bf16 workloads), b [t] [hidden] hidden bias, w [t]
    [hidden] output weights, c [t] output bias."""
    a: np.ndarray
    b: np.ndarray
    w: np.ndarray
    c: np.ndarray


HEAD_TASKS, HEAD_HIDDEN = 4, 256


def head_weights(d_model: int, tasks: int = HEAD_TASKS, hidden: int = HEAD_HIDDEN, seed: int = 0,
                 dtype: str = "bf16") -> HeadWeights:
    """Seeded synthetic head weights: N(0, 1/d) first layer (unit-scale hidden
    pre-activations for unit-scale rows), N(0, 0.01) biases, N(0, 1/hidden)
    output weights."""
    rng = np.random.default_rng([seed, 0x4EAD])
    rnd = round_bf16 if dtype == "bf16" else (lambda a: a.astype(np.float32))
    a = rnd(rng.standard_normal((tasks, d_model, hidden)) / np.sqrt(d_model))
    b = (rng.standard_normal((tasks, hidden)) * 0.1).astype(np.float32)
    w = (rng.standard_normal((tasks, hidden)) / np.sqrt(hidden)).astype(np.float32)
    c = (rng.standard_normal(tasks) * 0.1).astype(np.float32)
    return HeadWeights(a, b, w, c)


@dataclass
class Workload:
    cfg: Config
    seed: int
    user_ids: np.ndarray        # [B] int64, batch order
    hist_len: np.ndarray        # [B] int32 history tokens n_h
    n_targets: np.ndarray       # [B] int32 candidate tokens T
    hit: np.ndarray             # [B] bool: history cached before the request
    stale_ids: np.ndarray       # [S] int64 users cached before the request, not in the batch
    stale_hist_len: np.ndarray  # [S] int32
    prefill_order: np.ndarray   # indices into concat(batch users that hit, stale users): pre-fill order
    layers: List[LayerWeights]
    x: List[np.ndarray]         # per batch user [n_h + T, d] float32: history then candidates
    x_stale: List[np.ndarray]   # per stale user [n_h, d]
    num_pages: int
    page_perm: np.ndarray       # [num_pages] int32, initial free-queue order

    @property
    def seq_len(self) -> np.ndarray:
        return self.hist_len + self.n_targets


def _pages(n, p):
    return (int(n) + p - 1) // p


def _draw_lengths(rng, cfg: Config, n: int) -> np.ndarray:
    kind = cfg.hist[0]
    if kind == "fixed":
        vals = np.asarray(cfg.hist[1], dtype=np.int64)
        assert len(vals) == n
        return vals.astype(np.int32)
    if kind == "uniform":
        lo, hi = cfg.hist[1], cfg.hist[2]
        return rng.integers(lo, hi + 1, size=n).astype(np.int32)
    if kind == "lognormal":
        med, lo, hi = cfg.hist[1], cfg.hist[2], cfg.hist[3]
        z = rng.standard_normal(n)
        return np.clip(np.rint(med * np.exp(z)), lo, hi).astype(np.int32)
    raise ValueError(kind)


def pool_pages(cfg: Config, hist_len, n_targets, stale_hist_len) -> int:
    """Physical pages in the pool: what the batch needs after its append; for a
    mixed cache, plus half the stale users' pages (so eviction must run)."""
    p = cfg.page_size
    need = sum(_pages(h + t, p) for h, t in zip(hist_len, n_targets))
    if cfg.cache == "mixed":
        need += sum(_pages(h, p) for h in stale_hist_len) // 2
    return int(need)


def generate(cfg, seed: int = 0, *, batch: Optional[int] = None,
             hist_override: Optional[List[int]] = None) -> Workload:
    """Draw one workload.  `batch`/`hist_override` shrink a workload for tests
    (the draw order is unchanged)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if batch is not None:
        cfg = dataclasses.replace(cfg, batch=batch)
    rng = np.random.Generator(np.random.PCG64(seed))
    B = cfg.batch
    if hist_override is not None:
        hist = np.asarray(hist_override, dtype=np.int32)
        assert len(hist) == B
        if cfg.hist[0] != "fixed":
            _draw_lengths(rng, cfg, B)  # keep the draw order
    else:
        hist = _draw_lengths(rng, cfg, B)
    T = cfg.n_targets
    if cfg.hist[0] == "fixed" and T == 0:
        pass
    n_targets = np.full(B, T, dtype=np.int32)

    if cfg.cache == "mixed":
        n_hit = int(round(cfg.hit_fraction * B))
        hit = np.zeros(B, dtype=bool)
        hit[rng.permutation(B)[:n_hit]] = True
        stale_hist = _draw_lengths(rng, cfg, cfg.n_stale)
    elif cfg.cache == "hit":
        hit = np.ones(B, dtype=bool)
        stale_hist = np.zeros(0, dtype=np.int32)
    else:
        hit = np.zeros(B, dtype=bool)
        stale_hist = np.zeros(0, dtype=np.int32)
    S = len(stale_hist)

    ids = (rng.permutation(B + S) + 1).astype(np.int64) * 7 + 100
    user_ids, stale_ids = ids[:B], ids[B:]
    n_cached_before = int(hit.sum()) + S
    prefill_order = rng.permutation(n_cached_before).astype(np.int32)

    d, inner = cfg.d_model, cfg.inner
    rnd = round_bf16 if cfg.dtype == "bf16" else (lambda a: a.astype(np.float32))
    layers = []
    for _ in range(cfg.num_layers):
        w1 = rnd(rng.normal(0.0, 0.02, size=(d, 4 * inner)).astype(np.float32))
        w2 = rnd(rng.normal(0.0, 0.02, size=(inner, d)).astype(np.float32))
        rab = rnd(rng.normal(0.0, 0.1, size=(cfg.num_buckets,)).astype(np.float32))
        layers.append(LayerWeights(w1, w2, rab))
    x = [rnd(rng.standard_normal((int(hist[b]) + T, d)).astype(np.float32)) for b in range(B)]
    x_stale = [rnd(rng.standard_normal((int(stale_hist[s]), d)).astype(np.float32)) for s in range(S)]

    num_pages = pool_pages(cfg, hist, n_targets, stale_hist) if cfg.cache != "none" else 0
    page_perm = rng.permutation(num_pages).astype(np.int32)
    return Workload(cfg, seed, user_ids, hist, n_targets, hit, stale_ids, stale_hist,
                    prefill_order, layers, x, x_stale, num_pages, page_perm)


def workload_for(name: str, seed: int = 0, num_layers: Optional[int] = None, **kw) -> Workload:
    """Workload by name; a workload that shares another's data draws with its
    seed and config.  num_layers: the same workload with a deeper or shallower
    stack (the layers are drawn before the inputs, so the inputs differ)."""
    cfg = CONFIGS[name]
    if num_layers is not None:
        cfg = dataclasses.replace(cfg, num_layers=num_layers)
    if cfg.seed_alias is not None:
        base = CONFIGS[cfg.seed_alias]
        if num_layers is not None:
            base = dataclasses.replace(base, num_layers=num_layers)
        w = generate(base, seed, **kw)
        hist, T = w.hist_len, w.n_targets
        cfg2 = cfg if kw.get("batch") is None else dataclasses.replace(cfg, batch=kw["batch"])
        w.cfg = cfg2
        w.hit = np.ones(len(hist), dtype=bool)
        w.num_pages = pool_pages(cfg2, hist, T, w.stale_hist_len)
        prng = np.random.Generator(np.random.PCG64(seed + 0x5EED))
        w.prefill_order = prng.permutation(len(hist)).astype(np.int32)
        w.page_perm = prng.permutation(w.num_pages).astype(np.int32)
        return w
    return generate(cfg, seed, **kw)


def small_config(dtype="bf16", d_model=None, num_heads=2, head_dim=128, num_layers=1,
                 n_targets=0, cache="none", page_size=32, num_buckets=64, name="small"):
    """A reduced workload shape for tests (fixed lengths are passed to generate())."""
    d = d_model if d_model is not None else num_heads * head_dim
    return Config(name, dtype, 1, d, num_heads, head_dim, num_layers, ("uniform", 1, 1),
                  n_targets, cache, page_size=page_size, num_buckets=num_buckets)

"""Drive HSTU requests through libhstu with torch device memory and streams.

A request ("Deploying an HSTU Generative Recommender with NVIDIA
Dynamo-Triton", KV cache section): look the users up in the paged KV table,
evict least-recently-used users if pages are short, allocate room for the new
tokens, then run the layer stack on the new tokens only; every layer appends
its K/V of the new tokens and its attention reads cached history straight from
the pages.  Without a cache the same stack runs on contiguous K/V.

torch only allocates device buffers and supplies the stream; every arithmetic
step is a libhstu kernel.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import hstu
from .hstu import HSTU_BF16, HSTU_F32


def tdtype(dtype: int) -> torch.dtype:
    return torch.bfloat16 if dtype == HSTU_BF16 else torch.float32


def dtype_code(name: str) -> int:
    return HSTU_BF16 if name == "bf16" else HSTU_F32


def stream_handle(stream: Optional[torch.cuda.Stream] = None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("libhstu needs a GPU (gfx950); none is visible")
    hstu.lib()


class Model:
    """Device copies of a stack's weights in the library's output-major layout
    (w1 = W1^T [4*H*dh][d], w2 = W2^T [d][H*dh], for x . W1 and g . W2) in the
    compute dtype, and rab [num_buckets] fp32, per layer."""

    def __init__(self, layers, dtype: int, num_heads: int, head_dim: int, d_model: int,
                 eps: float = 1e-5, device="cuda"):
        self.dtype, self.num_heads, self.head_dim, self.d_model, self.eps = dtype, num_heads, head_dim, d_model, eps
        t = tdtype(dtype)
        self.w1 = [torch.from_numpy(np.ascontiguousarray(lw.w1.T)).to(device=device, dtype=t) for lw in layers]
        self.w2 = [torch.from_numpy(np.ascontiguousarray(lw.w2.T)).to(device=device, dtype=t) for lw in layers]
        self.rab = [torch.from_numpy(np.ascontiguousarray(lw.rab, dtype=np.float32)).to(device) for lw in layers]
        # W1 [d][4 H dh] and W2 [H dh][d] in the layout of x . W1 and g . W2 (the backward's operands)
        self.w1t = [w.t().contiguous() for w in self.w1]
        self.w2t = [w.t().contiguous() for w in self.w2]
        # W1's column sums, computed once for the bf16 layer's fused pre-norm
        self.w1_colsum = [None] * len(self.w1)
        if dtype == HSTU_BF16 and str(device).startswith("cuda"):
            for li, w in enumerate(self.w1):
                cs = torch.empty(w.shape[0], dtype=torch.float32, device=device)
                hstu.hstu_w1_colsum(w.data_ptr(), w.shape[0], w.shape[1], cs.data_ptr(), stream_handle())
                self.w1_colsum[li] = cs

    @property
    def num_layers(self) -> int:
        return len(self.w1)


class PagedCache:
    """K/V pools [layers][pages][H][P][dh] in device memory plus the library's
    host metadata handle."""

    def __init__(self, num_layers, num_heads, head_dim, page_size, num_pages, dtype: int,
                 free_order=None, device="cuda", zero=True):
        n = num_layers * num_pages * num_heads * page_size * head_dim
        alloc = torch.zeros if zero else torch.empty
        self.k_pool = alloc(max(n, 1), dtype=tdtype(dtype), device=device)
        self.v_pool = alloc(max(n, 1), dtype=tdtype(dtype), device=device)
        self.num_layers, self.num_heads, self.head_dim = num_layers, num_heads, head_dim
        self.page_size, self.num_pages, self.dtype = page_size, num_pages, dtype
        self.h = hstu.kv_cache_create(num_layers, num_heads, head_dim, page_size, num_pages, dtype,
                                      self.k_pool.data_ptr(), self.v_pool.data_ptr(), free_order)
        self.host_pages = 0
        self.host_k = self.host_v = None

    def attach_host(self, host_pages: int):
        """A host tier of host_pages pages of the same geometry, its pools in
        pinned host memory; users evicted for room are then offloaded to it
        and onboarded again when they are requested."""
        n = self.num_layers * host_pages * self.num_heads * self.page_size * self.head_dim
        self.host_k = torch.zeros(max(n, 1), dtype=tdtype(self.dtype), pin_memory=True)
        self.host_v = torch.zeros(max(n, 1), dtype=tdtype(self.dtype), pin_memory=True)
        hstu.kv_host_attach(self.h, host_pages, self.host_k.data_ptr(), self.host_v.data_ptr())
        self.host_pages = host_pages

    def __del__(self):
        if getattr(self, "h", None):
            hstu.lib().kv_cache_destroy(self.h)
            self.h = None

    def pages_needed(self, cached_len, n_new) -> int:
        P = self.page_size
        return int(sum(-(-(c + t) // P) - (-(-c // P)) for c, t in zip(cached_len, n_new)))


@dataclass
class Request:
    users: np.ndarray
    new_len: np.ndarray
    cached_len: np.ndarray
    n_targets: np.ndarray
    norm_n: np.ndarray
    kv_len: np.ndarray
    plan: int
    info: hstu.hstu_plan_info
    meta: torch.Tensor
    page_table: Optional[torch.Tensor]
    max_pages: int
    evicted: np.ndarray
    num_heads: int = 1
    head_dim: int = 128
    offloaded: np.ndarray = None      # users moved to the host tier to make room
    host_dropped: np.ndarray = None   # host-tier users dropped to make room there
    onboarded: np.ndarray = None      # requested users brought back from the host tier

    def close(self):
        if self.plan:
            hstu.hstu_plan_destroy(self.plan)
            self.plan = 0


class RequestBuffers:
    """Device buffers a stream of requests reuses (page table, plan metadata)
    and pinned staging for the page-table upload, so that preparing request
    k+1 on the host never waits for request k on the GPU.  Uploads are
    ordered on the stream, so reusing the device buffers is safe."""

    def __init__(self, max_batch: int, max_pages: int, meta_bytes: int = 1 << 20, device="cuda", slots: int = 3):
        self.max_batch, self.max_pages = max_batch, max(max_pages, 1)
        n = max_batch * self.max_pages
        self.d_pt = torch.empty(max(n, 1), dtype=torch.int32, device=device)
        self.d_meta = torch.empty(max(meta_bytes, 256), dtype=torch.uint8, device=device)
        self.pinned = [torch.empty(max(n, 1), dtype=torch.int32, pin_memory=True) for _ in range(slots)]
        self.events = [None] * slots
        self.slot = 0

    def upload_page_table(self, pt: np.ndarray) -> torch.Tensor:
        n = pt.size
        k = self.slot
        self.slot = (self.slot + 1) % len(self.pinned)
        if self.events[k] is not None:
            while not self.events[k].query():  # poll: a blocking wait can oversleep
                pass
        self.pinned[k][:n].numpy()[:] = pt.reshape(-1)
        dst = self.d_pt[:n]
        dst.copy_(self.pinned[k][:n], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self.events[k] = ev
        return dst.view(pt.shape)

    def meta(self, nbytes: int, device="cuda") -> torch.Tensor:
        if nbytes > self.d_meta.numel():
            self.d_meta = torch.empty(2 * nbytes, dtype=torch.uint8, device=device)
        return self.d_meta


def prepare(cache: Optional[PagedCache], users, new_len, n_targets, norm_n=None, max_pages: int = 0,
            num_heads: int = 1, head_dim: int = 128, device="cuda", stream=None,
            bufs: Optional[RequestBuffers] = None) -> Request:
    """Host cache operations (lookup, LRU eviction, allocation), page-table
    upload, and the request plan, uploaded (asynchronously when `bufs` is
    given).  With a host tier, requested users found there are onboarded
    (their cached length counts as a hit), and the LRU victims that make room
    are offloaded to it rather than dropped (dropped only if the host tier
    cannot take them); the page copies go on the request's stream."""
    users = np.asarray(users, np.int64)
    new_len = np.asarray(new_len, np.int32)
    n_targets = np.asarray(n_targets, np.int32)
    s = stream_handle(stream)
    evicted = offloaded = host_dropped = onboarded = np.zeros(0, np.int64)
    if cache is not None:
        cached = hstu.kv_lookup(cache.h, users)
        need = cache.pages_needed(cached, new_len)
        if cache.host_pages:
            where, host_len = hstu.kv_residency(cache.h, users)
            on_host = where == 2
            onboarded = users[on_host]
            cached = np.where(on_host, host_len, cached).astype(np.int32)
            need = cache.pages_needed(cached, new_len) + sum(_ceil(c, cache.page_size) for c in cached[on_host])
        if hstu.kv_free_pages(cache.h) < need:
            if cache.host_pages:
                # the step after choosing LRU victims: keep their pages on the host tier
                victims = hstu.kv_lru_victims(cache.h, need, users)
                try:
                    host_dropped = hstu.kv_offload(cache.h, victims, s, pinned=onboarded)
                    offloaded = victims
                except hstu.HstuError as e:
                    if e.status != hstu.HSTU_ERR_NO_SPACE:
                        raise
                    evicted = hstu.kv_evict_lru(cache.h, need, users)
            else:
                evicted = hstu.kv_evict_lru(cache.h, need, users)
        if len(onboarded):
            hstu.kv_onboard(cache.h, onboarded, s)
        pt, kv_len = hstu.kv_page_alloc(cache.h, users, new_len, max_pages)
        d_pt = bufs.upload_page_table(pt) if bufs is not None else torch.from_numpy(pt).to(device)
        page_size, num_heads, head_dim = cache.page_size, cache.num_heads, cache.head_dim
    else:
        cached = np.zeros(len(users), np.int32)
        kv_len = new_len.copy()
        d_pt, page_size, max_pages = None, 0, 0
    nn = (cached + new_len).astype(np.float32) if norm_n is None else np.asarray(norm_n, np.float32)
    plan = hstu.hstu_plan_create(num_heads, head_dim, new_len, cached, n_targets, nn, page_size, max_pages)
    info = hstu.hstu_plan_get_info(plan)
    if bufs is not None:
        meta = bufs.meta(int(info.meta_bytes), device)
    else:
        meta = torch.empty(max(int(info.meta_bytes), 256), dtype=torch.uint8, device=device)
    hstu.hstu_plan_upload(plan, meta.data_ptr(), meta.numel(), s)
    return Request(users, new_len, np.asarray(cached, np.int32), n_targets, nn, np.asarray(kv_len, np.int32),
                   plan, info, meta, d_pt, max_pages, evicted, num_heads, head_dim, offloaded, host_dropped,
                   onboarded)


def layer_args(model: Model, req: Request, li: int, x: torch.Tensor, y: torch.Tensor,
               cache: Optional[PagedCache], workspace: Optional[torch.Tensor] = None,
               taps: Optional[dict] = None) -> hstu.hstu_layer_args:
    a = hstu.hstu_layer_args()
    a.dtype = model.dtype
    a.d_model = model.d_model
    a.eps = model.eps
    a.plan = req.plan
    a.x = x.data_ptr()
    a.y = y.data_ptr()
    a.w1 = model.w1[li].data_ptr()
    a.w2 = model.w2[li].data_ptr()
    a.rab = model.rab[li].data_ptr()
    a.num_buckets = model.rab[li].numel()
    if model.w1_colsum[li] is not None:
        a.w1_colsum = model.w1_colsum[li].data_ptr()
    if cache is not None:
        a.cache = cache.h
        a.layer = li
        a.d_page_table = req.page_table.data_ptr()
    if taps:
        a.uvqk_out = taps["uvqk"].data_ptr() if "uvqk" in taps else None
        a.o_out = taps["o"].data_ptr() if "o" in taps else None
        a.g_out = taps["g"].data_ptr() if "g" in taps else None
        a.s_out = taps["s"].data_ptr() if "s" in taps else None
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel()
    return a


def _layer_ws_bytes(model: Model, req: Request) -> int:
    a = hstu.hstu_layer_args()
    a.dtype, a.d_model, a.plan = model.dtype, model.d_model, req.plan
    return hstu.hstu_layer_workspace_size(a)


def _stats_bytes(model: Model, n_new: int) -> int:
    """One buffer of row statistics that f2 hands to the next layer's pre-norm
    (bf16, d_model <= 512): [n_new][d_model / 128] (mean, M2) pairs; the rows'
    pool slots (int64 [n_new]) take no more."""
    if model.dtype != hstu.HSTU_BF16 or model.d_model > 512:
        return 0
    return -(-(n_new * max(model.d_model // 128, 1) * 8) // 256) * 256


def workspace_for(model: Model, req: Request, device="cuda") -> torch.Tensor:
    """The layer workspace followed by two row-statistics buffers (ping-pong
    between the layers of a stack) and the rows' pool slots."""
    n = _layer_ws_bytes(model, req) + 3 * _stats_bytes(model, int(req.info.n_new_total))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def forward(model: Model, req: Request, x: torch.Tensor, cache: Optional[PagedCache],
            workspace: Optional[torch.Tensor] = None, layers: Optional[Sequence[int]] = None,
            taps: Optional[List[dict]] = None, stream=None,
            out_bufs: Optional[List[torch.Tensor]] = None) -> torch.Tensor:
    """Runs the stack on the new tokens x [N_new, d] in one native call
    (hstu_stack_forward); layer k writes out_bufs[k % len(out_bufs)] (two
    buffers by default) and the last layer's y is returned.  Each layer's f2
    leaves the row statistics of its y for the next layer's pre-norm when the
    workspace has room for them."""
    s = stream_handle(stream)
    if workspace is None:
        workspace = workspace_for(model, req, x.device)
    layers = list(range(model.num_layers)) if layers is None else list(layers)
    if out_bufs is None:
        out_bufs = [torch.empty_like(x), torch.empty_like(x)]
    lw, sb = _layer_ws_bytes(model, req), _stats_bytes(model, x.shape[0])
    stats = None
    if sb and len(layers) > 1 and workspace.numel() >= lw + 3 * sb:
        base = workspace.data_ptr() + lw
        stats = [base, base + sb, base + 2 * sb]   # y/x statistics ping-pong, pool slots
    cur = x
    args = []
    for k, li in enumerate(layers):
        out = out_bufs[k % len(out_bufs)]
        a = layer_args(model, req, li, cur, out, cache, workspace, taps[k] if taps else None)
        if stats is not None:
            a.workspace_bytes = lw
            a.row_slots = stats[2]
            if k > 0:
                a.x_stats = stats[(k - 1) % 2]
            if k + 1 < len(layers):
                a.y_stats = stats[k % 2]
        args.append(a)
        cur = out
    hstu.hstu_stack_forward(args, s)
    return cur


def forward_for_backward(model: Model, req: Request, x: torch.Tensor, stream=None):
    """The stack on x (contiguous keys, no cache), one layer at a time,
    keeping what the backward reuses: per layer its input and the uvqk, s
    and o taps.  Returns (y, saved)."""
    inner = model.num_heads * model.head_dim
    n = x.shape[0]
    t = tdtype(model.dtype)
    ws = workspace_for(model, req, x.device)
    saved, cur = [], x
    for li in range(model.num_layers):
        taps = {"uvqk": torch.empty((n, 4 * inner), dtype=t, device=x.device),
                "s": torch.empty((n, 4 * inner), dtype=t, device=x.device),
                "o": torch.empty((n, inner), dtype=torch.float32, device=x.device)}
        y = forward(model, req, cur, None, ws, layers=[li], taps=[taps], stream=stream,
                    out_bufs=[torch.empty_like(cur)])
        saved.append(dict(x=cur, **taps))
        cur = y
    return cur, saved


def backward(model: Model, req: Request, saved, dy: torch.Tensor, stream=None,
             workspace: Optional[torch.Tensor] = None, stop_at: int = 0):
    """hstu_layer_backward from the last layer down to layer stop_at.  Returns
    (dL/d(input of layer stop_at), per-layer dict of dw1 [4 H dh][d],
    dw2 [d][H dh], drab [nb], all fp32 in the forward's weight layouts)."""
    s = stream_handle(stream)
    grads = [None] * model.num_layers
    cur = dy
    for li in reversed(range(stop_at, model.num_layers)):
        sv = saved[li]
        g = {"dw1": torch.empty(model.w1[li].shape, dtype=torch.float32, device=dy.device),
             "dw2": torch.empty(model.w2[li].shape, dtype=torch.float32, device=dy.device),
             "drab": torch.empty(model.rab[li].shape, dtype=torch.float32, device=dy.device)}
        dx = torch.empty_like(cur)
        a = hstu.hstu_layer_bwd_args()
        a.dtype, a.d_model, a.eps, a.plan = model.dtype, model.d_model, model.eps, req.plan
        a.x, a.w1t, a.w2t = sv["x"].data_ptr(), model.w1t[li].data_ptr(), model.w2t[li].data_ptr()
        a.rab, a.num_buckets = model.rab[li].data_ptr(), model.rab[li].numel()
        a.uvqk, a.s, a.o = sv["uvqk"].data_ptr(), sv["s"].data_ptr(), sv["o"].data_ptr()
        a.dy, a.dx = cur.data_ptr(), dx.data_ptr()
        a.dw1, a.dw2, a.drab = g["dw1"].data_ptr(), g["dw2"].data_ptr(), g["drab"].data_ptr()
        need = hstu.hstu_layer_backward_workspace_size(a)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dy.device)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
        hstu.hstu_layer_backward(a, s)
        grads[li] = g
        cur = dx
    return cur, grads


class Head:
    """Device copies of a multitask ranking head in the library's layout:
    w_hidden output-major [tasks*hidden][d] (row t*hidden + j = task t's
    column j), b_hidden and w_out flat fp32 [tasks*hidden], b_out [tasks]."""

    def __init__(self, hw, dtype: int, device="cuda"):
        tasks, d, hidden = hw.a.shape
        self.dtype, self.tasks, self.hidden, self.d_model = dtype, tasks, hidden, d
        wt = np.ascontiguousarray(np.transpose(hw.a, (0, 2, 1)).reshape(tasks * hidden, d))
        self.w_hidden = torch.from_numpy(wt).to(device=device, dtype=tdtype(dtype))
        self.b_hidden = torch.from_numpy(np.ascontiguousarray(hw.b, np.float32).reshape(-1)).to(device)
        self.w_out = torch.from_numpy(np.ascontiguousarray(hw.w, np.float32).reshape(-1)).to(device)
        self.b_out = torch.from_numpy(np.ascontiguousarray(hw.c, np.float32)).to(device)
        self.workspace = torch.empty(256, dtype=torch.uint8, device=device)

    def args(self, y: torch.Tensor, rows: torch.Tensor, n_rows: int, logits: torch.Tensor) -> hstu.hstu_head_args:
        a = hstu.hstu_head_args()
        a.dtype, a.d_model, a.num_tasks, a.hidden = self.dtype, self.d_model, self.tasks, self.hidden
        a.y, a.y_rows = y.data_ptr(), y.shape[0]
        a.d_rows, a.n_rows = rows.data_ptr(), n_rows
        a.w_hidden, a.b_hidden = self.w_hidden.data_ptr(), self.b_hidden.data_ptr()
        a.w_out, a.b_out, a.logits = self.w_out.data_ptr(), self.b_out.data_ptr(), logits.data_ptr()
        need = hstu.hstu_head_workspace_size(a)
        if need > self.workspace.numel():
            self.workspace = torch.empty(2 * need, dtype=torch.uint8, device=y.device)
        a.workspace, a.workspace_bytes = self.workspace.data_ptr(), self.workspace.numel()
        return a

    def __call__(self, y: torch.Tensor, rows: torch.Tensor, n_rows: Optional[int] = None, stream=None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Logits [n_rows, tasks] fp32 of rows `rows` (device int32) of y."""
        n = rows.numel() if n_rows is None else n_rows
        logits = out if out is not None else torch.empty((max(n, 1), self.tasks), dtype=torch.float32,
                                                         device=y.device)
        hstu.hstu_head_forward(self.args(y, rows, n, logits), stream_handle(stream))
        return logits[:n]


def candidate_row_list(new_len, n_targets) -> np.ndarray:
    """The new-token rows of each user's candidates: its last min(T_u, t_u)
    new tokens, users in batch order."""
    ends = np.cumsum(np.asarray(new_len, np.int64))
    take = np.minimum(np.asarray(n_targets, np.int64), np.asarray(new_len, np.int64))
    parts = [np.arange(e - t, e) for e, t in zip(ends, take)]
    return np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)


def attention(req: Request, q: torch.Tensor, q_row_stride: int, rab: torch.Tensor, dtype: int,
              k: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None, kv_row_stride: int = 0,
              cache: Optional[PagedCache] = None, layer: int = 0, stream=None,
              static_scratch: bool = False, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_attn_fwd: o [N_new, H*dh] fp32 (includes 1/n).  static_scratch:
    hstu_attn_fwd_static instead (partial tiles in the library's static
    device array; no workspace)."""
    s = stream_handle(stream)
    H, dh = req.num_heads, req.head_dim
    if out is None:
        out = torch.empty((int(req.info.n_new_total), H * dh), dtype=torch.float32, device=q.device)
    ws = None if static_scratch else torch.empty(max(int(req.info.attn_workspace_bytes), 256), dtype=torch.uint8,
                                                  device=q.device)
    a = hstu.hstu_attn_args()
    a.dtype = dtype
    a.plan = req.plan
    a.q = q.data_ptr()
    a.q_row_stride = q_row_stride
    if cache is not None:
        a.cache = cache.h
        a.layer = layer
        a.d_page_table = req.page_table.data_ptr()
    else:
        a.k, a.v, a.kv_row_stride = k.data_ptr(), v.data_ptr(), kv_row_stride
    a.rab = rab.data_ptr()
    a.num_buckets = rab.numel()
    a.out = out.data_ptr()
    if static_scratch:
        hstu.hstu_attn_fwd_static(a, s)
    else:
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel()
        hstu.hstu_attn_fwd(a, s)
    return out


def prepare_attn(cache, users, new_len, n_targets, norm_n, max_pages, num_heads, head_dim, cached_len=None,
                 device="cuda"):
    """A plan for hstu_attn_fwd alone.  With a cache the page table comes from
    the cache (positions must already be there); without one, cached_len gives
    the contiguous prefix length of each user."""
    new_len = np.asarray(new_len, np.int32)
    n_targets = np.asarray(n_targets, np.int32)
    s = stream_handle()
    if cache is not None:
        pt, kv_len = hstu.kv_page_table(cache.h, users, max_pages)
        cached = (kv_len - new_len).astype(np.int32)
        d_pt = torch.from_numpy(pt).to(device)
        page_size = cache.page_size
    else:
        cached = np.zeros(len(new_len), np.int32) if cached_len is None else np.asarray(cached_len, np.int32)
        kv_len = cached + new_len
        d_pt, page_size, max_pages = None, 0, 0
    nn = kv_len.astype(np.float32) if norm_n is None else np.asarray(norm_n, np.float32)
    plan = hstu.hstu_plan_create(num_heads, head_dim, new_len, cached, n_targets, nn, page_size, max_pages)
    info = hstu.hstu_plan_get_info(plan)
    meta = torch.empty(max(int(info.meta_bytes), 256), dtype=torch.uint8, device=device)
    hstu.hstu_plan_upload(plan, meta.data_ptr(), meta.numel(), s)
    return Request(np.asarray(users, np.int64), new_len, cached, n_targets, nn, np.asarray(kv_len, np.int32),
                   plan, info, meta, d_pt, max_pages, np.zeros(0, np.int64), num_heads, head_dim)


# ---------------------------------------------------------------------------
# a workload's serving scenario: weights, pool, pre-filled cache, request
# ---------------------------------------------------------------------------

def _ceil(a, b):
    return -(-int(a) // int(b))


class Scenario:
    """Device state for one synthetic workload.

    cache "none":  every request recomputes each user's whole sequence.
    cache "hit":   each user's history is pre-filled into the pages (placed by
                   the workload's page permutation); the request computes and
                   appends only the candidates.
    cache "mixed": hit users and stale users are pre-filled; the request runs
                   hit users on their candidates and the others on their whole
                   sequence, evicting least-recently-used stale users.
    Pre-fill uses the final normaliser n_u = history + candidates, so a cached
    prefix plus the appended candidates equals a full recompute."""

    def __init__(self, w, device="cuda"):
        self.w, self.cfg, self.device = w, w.cfg, device
        cfg = w.cfg
        self.dtype = dtype_code(cfg.dtype)
        self.model = Model(w.layers, self.dtype, cfg.num_heads, cfg.head_dim, cfg.d_model, cfg.eps, device)
        L = w.hist_len + w.n_targets
        lens = list(L) + [int(h) + cfg.n_targets for h in w.stale_hist_len]
        self.max_pages = max(1, max(_ceil(l, cfg.page_size) for l in lens)) if lens else 1
        self.cache = None
        if cfg.cache != "none":
            self.cache = PagedCache(cfg.num_layers, cfg.num_heads, cfg.head_dim, cfg.page_size, w.num_pages,
                                    self.dtype, w.page_perm, device)
        self.snapshot = None

    def _x(self, rows) -> torch.Tensor:
        a = np.concatenate(rows, axis=0) if rows else np.zeros((0, self.cfg.d_model), np.float32)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=self.device, dtype=tdtype(self.dtype))

    def prefill(self):
        """Pre-fills the cached users' histories (in the workload's pre-fill order)."""
        w, cfg = self.w, self.cfg
        if self.cache is None:
            return
        cached_users = [(w.user_ids[b], w.x[b][:w.hist_len[b]], int(w.hist_len[b] + w.n_targets[b]))
                        for b in range(cfg.batch) if w.hit[b]]
        cached_users += [(w.stale_ids[s], w.x_stale[s], int(w.stale_hist_len[s] + cfg.n_targets))
                         for s in range(len(w.stale_ids))]
        order = [cached_users[i] for i in w.prefill_order]
        if order:
            users = [u for u, _, _ in order]
            new_len = [len(x) for _, x, _ in order]
            req = prepare(self.cache, users, new_len, [0] * len(users), [n for _, _, n in order],
                          self.max_pages, device=self.device)
            forward(self.model, req, self._x([x for _, x, _ in order]), self.cache)
            torch.cuda.synchronize()
            req.close()
        self.snapshot = hstu.kv_state_dump(self.cache.h)

    def request_inputs(self):
        """(users, new_len, n_targets, norm_n, list of new-token rows) in batch order."""
        w = self.w
        users, new_len, rows = [], [], []
        for b in range(self.cfg.batch):
            x = w.x[b]
            start = int(w.hist_len[b]) if w.hit[b] else 0
            users.append(int(w.user_ids[b]))
            new_len.append(len(x) - start)
            rows.append(x[start:])
        norm_n = (w.hist_len + w.n_targets).astype(np.float32)
        return users, new_len, list(w.n_targets), norm_n, rows

    def restore(self):
        if self.cache is not None and self.snapshot is not None:
            hstu.kv_state_load(self.cache.h, self.snapshot)

    def make_request(self, x_rows=None):
        users, new_len, n_targets, norm_n, rows = self.request_inputs()
        req = prepare(self.cache, users, new_len, n_targets, norm_n, self.max_pages, self.cfg.num_heads,
                      self.cfg.head_dim, self.device)
        return req, self._x(rows if x_rows is None else x_rows)

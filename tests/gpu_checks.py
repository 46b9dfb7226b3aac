"""Helpers of the GPU parity tests: per-layer comparison of the HIP path with
the oracle, fed the GPU's own layer input and cache bytes so error does not
compound across layers.

Tolerance (per tensor, per layer): rel = max|gpu - ref| / max|ref| must stay
below 2e-2 in bf16 and 1e-4 in fp32, on O (attention output incl. 1/n), G
(LayerNorm(O) * U), Y, and the new K/V.  The branch Y - X is checked against
the same bound plus half a unit in the last place of Y's storage type: Y is
stored rounded (bf16 has 8 significant bits) and the residual X is about ten
times larger than the branch, so the storage rounding alone can exceed 2e-2
of the branch's maximum without any arithmetic error in the branch.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from generative_recommender_sequence_amd import runtime
from generative_recommender_sequence_amd.hstu import HSTU_BF16

TOL = {HSTU_BF16: 2e-2, 0: 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel(gpu, ref) -> float:
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / max(den, 1e-30))


def half_ulp(y: np.ndarray, dtype: int) -> np.ndarray:
    mant = 8 if dtype == HSTU_BF16 else 24
    e = np.floor(np.log2(np.maximum(np.abs(y), 1e-30)))
    return 2.0 ** (e - mant)


def branch_excess(y_gpu, y_ref, x, dtype, ulps: int = 1) -> float:
    """max(|(y_gpu - x) - (y_ref - x)| - ulps * half_ulp(y_ref)) / max|y_ref - x|
    (ulps = 2 when y_ref is itself a rounded stored value)"""
    br = y_ref - x
    err = np.abs(y_gpu - y_ref) - ulps * half_ulp(y_ref, dtype)
    return float(max(np.max(err), 0.0) / max(np.max(np.abs(br)), 1e-30)) if br.size else 0.0


def pool_rows(cache: runtime.PagedCache, which: str, layer: int, pt_row, start: int, stop: int) -> np.ndarray:
    """Positions [start, stop) of one user at `layer`, read from the pool on the
    device with plain torch indexing -> float64 [n, H*dh]."""
    pool = cache.k_pool if which == "k" else cache.v_pool
    H, P, dh = cache.num_heads, cache.page_size, cache.head_dim
    view = pool.view(cache.num_layers, cache.num_pages, H, P, dh)
    if stop <= start:
        return np.zeros((0, H * dh))
    pages = torch.as_tensor(np.asarray(pt_row[:(stop + P - 1) // P], np.int64), device=pool.device)
    rows = view[layer].index_select(0, pages).permute(0, 2, 1, 3).reshape(-1, H * dh)
    return to64(rows[start:stop])


def run_layers_with_taps(scn: runtime.Scenario, req, x: torch.Tensor):
    """Runs the stack in one call, as the product does (so each layer's
    pre-norm takes the row statistics the layer before left), with taps and
    one output buffer per layer; returns per-layer dicts of device tensors
    (x, y, uvqk, o, g)."""
    model = scn.model
    inner = model.num_heads * model.head_dim
    n = x.shape[0]
    t = runtime.tdtype(model.dtype)
    ws = runtime.workspace_for(model, req, x.device)
    taps = [{"uvqk": torch.empty((n, 4 * inner), dtype=t, device=x.device),
             "o": torch.empty((n, inner), dtype=torch.float32, device=x.device),
             "g": torch.empty((n, inner), dtype=t, device=x.device)} for _ in range(model.num_layers)]
    ys = [torch.empty_like(x) for _ in range(model.num_layers)]
    runtime.forward(model, req, x, scn.cache, ws, taps=taps, out_bufs=ys)
    torch.cuda.synchronize()
    xs = [x] + ys[:-1]
    return [dict(x=xs[li], y=ys[li], **taps[li]) for li in range(model.num_layers)]


def check_layers(scn: runtime.Scenario, req, per_layer, sample, label="") -> dict:
    """Per-layer oracle comparison on the users at batch indices `sample`.
    Returns the worst relative error per tensor."""
    cfg, model = scn.cfg, scn.model
    H, dh, inner = cfg.num_heads, cfg.head_dim, cfg.inner
    q_off = np.concatenate([[0], np.cumsum(req.new_len)])
    rows = np.concatenate([np.arange(q_off[b], q_off[b + 1]) for b in sample]).astype(np.int64)
    pt = req.page_table.cpu().numpy() if req.page_table is not None else None
    worst = {}
    for li, lay in enumerate(per_layer):
        t0 = time.time()
        x = to64(lay["x"])[rows]
        hist_k, hist_v = [], []
        for b in sample:
            c = int(req.cached_len[b])
            if c:
                hist_k.append(pool_rows(scn.cache, "k", li, pt[b], 0, c))
                hist_v.append(pool_rows(scn.cache, "v", li, pt[b], 0, c))
        hk = np.concatenate(hist_k) if hist_k else np.zeros((0, inner))
        hv = np.concatenate(hist_v) if hist_v else np.zeros((0, inner))
        ref = oracle.layer(x, model_w(scn, li, "w1"), model_w(scn, li, "w2"), scn.w.layers[li].rab,
                           req.new_len[sample], req.cached_len[sample], req.n_targets[sample],
                           req.norm_n[sample], hk, hv, H, dh, cfg.eps)
        uvqk = to64(lay["uvqk"])[rows]
        got = {"o": to64(lay["o"])[rows], "g": to64(lay["g"])[rows], "y": to64(lay["y"])[rows],
               "u": uvqk[:, :inner], "v": uvqk[:, inner:2 * inner], "q": uvqk[:, 2 * inner:3 * inner],
               "k": uvqk[:, 3 * inner:]}
        errs = {k: rel(got[k], ref[k]) for k in got}
        errs["y-x"] = branch_excess(got["y"], ref["y"], x, scn.dtype)
        if scn.cache is not None:
            kk, vv = [], []
            for b in sample:
                c, L = int(req.cached_len[b]), int(req.kv_len[b])
                kk.append(pool_rows(scn.cache, "k", li, pt[b], c, L))
                vv.append(pool_rows(scn.cache, "v", li, pt[b], c, L))
            errs["k_pool"] = rel(np.concatenate(kk), ref["k"])
            errs["v_pool"] = rel(np.concatenate(vv), ref["v"])
        say(f"  {label} layer {li}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) +
            f"  (oracle {time.time() - t0:.1f}s)")
        for k, v in errs.items():
            worst[k] = max(worst.get(k, 0.0), v)
    return worst


def model_w(scn, li, name):
    return getattr(scn.w.layers[li], name)

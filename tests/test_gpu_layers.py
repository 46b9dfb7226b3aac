"""GPU parity of hstu_layer_forward against the oracle, layer by layer, on
small jagged batches (fp32 and bf16, with and without the paged cache), and
the cache invariant on the GPU: a cached prefix plus the appended candidates
gives the same outputs as a full recompute."""
import dataclasses

import numpy as np
import pytest
import torch

from generative_recommender_sequence_amd import hstu, runtime
from generative_recommender_sequence_amd.workloads import CONFIGS, generate, round_bf16, small_config
from gpu_checks import TOL, check_layers, rel, run_layers_with_taps, say, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    runtime.require_gpu()


def _assert_within(worst, tol):
    bad = {k: v for k, v in worst.items() if not v < tol}
    assert not bad, f"over tolerance {tol}: {bad}"


def test_c1_layer_fp32():
    say("C1 fp32 layer")
    w = generate(CONFIGS["C1"], 0)
    scn = runtime.Scenario(w)
    req, x = scn.make_request()
    per = run_layers_with_taps(scn, req, x)
    worst = check_layers(scn, req, per, [0, 1], "C1")
    _assert_within(worst, TOL[scn.dtype])
    req.close()


def _small(cache, dtype, hist, T, layers=2, H=2, P=32, seed=0, hit=None):
    cfg = small_config(dtype=dtype, num_heads=H, head_dim=128 if dtype == "bf16" else 64,
                       num_layers=layers, n_targets=T, cache=cache, page_size=P)
    w = generate(cfg, seed, batch=len(hist), hist_override=list(hist))
    if cache != "none":
        w.hit = np.ones(len(hist), bool) if hit is None else np.asarray(hit)
        w.prefill_order = np.arange(int(w.hit.sum()), dtype=np.int32)
        w.num_pages = sum(-(-int(h + T) // P) for h in hist) + 5
        w.page_perm = np.random.default_rng(seed + 1).permutation(w.num_pages).astype(np.int32)
        w.cfg = dataclasses.replace(cfg, batch=len(hist))
    # O(1) activations so every term matters
    for lw in w.layers:
        lw.w1 *= 4.0
        lw.w2 *= 4.0
    return w


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layers_no_cache(dtype):
    say(f"small no-cache {dtype}")
    w = _small("none", dtype, hist=[1, 70, 300, 129], T=5)
    scn = runtime.Scenario(w)
    req, x = scn.make_request()
    per = run_layers_with_taps(scn, req, x)
    worst = check_layers(scn, req, per, [0, 1, 2, 3], f"nocache-{dtype}")
    _assert_within(worst, TOL[scn.dtype])
    req.close()


@pytest.mark.parametrize("dtype,P", [("f32", 16), ("bf16", 32), ("bf16", 64)])
def test_layers_cached_candidates(dtype, P):
    say(f"small cached {dtype} P={P}")
    w = _small("hit", dtype, hist=[200, 33, 1000], T=64, P=P, hit=[True, True, True])
    scn = runtime.Scenario(w)
    scn.prefill()
    req, x = scn.make_request()
    per = run_layers_with_taps(scn, req, x)
    worst = check_layers(scn, req, per, [0, 1, 2], f"cached-{dtype}")
    _assert_within(worst, TOL[scn.dtype])
    req.close()


def test_layers_mixed_hit_and_miss_bf16():
    say("small mixed hit/miss bf16")
    w = _small("hit", "bf16", hist=[500, 90, 260], T=16, hit=[True, False, True])
    scn = runtime.Scenario(w)
    scn.prefill()
    req, x = scn.make_request()
    per = run_layers_with_taps(scn, req, x)
    worst = check_layers(scn, req, per, [0, 1, 2], "mixed")
    _assert_within(worst, 2e-2)
    req.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cached_prefix_plus_append_equals_full_recompute(dtype):
    say(f"cache invariant {dtype}")
    hist, T = [300, 77, 1200], 32
    w = _small("hit", dtype, hist=hist, T=T, layers=3)
    w_full = dataclasses.replace(w, cfg=dataclasses.replace(w.cfg, cache="none"), hit=np.zeros(3, bool))
    full = runtime.Scenario(w_full)
    req_f, x_f = full.make_request()
    y_full = to64(runtime.forward(full.model, req_f, x_f, None))
    cached = runtime.Scenario(w)
    cached.prefill()
    req_c, x_c = cached.make_request()
    y_c = to64(runtime.forward(cached.model, req_c, x_c, cached.cache))
    torch.cuda.synchronize()
    off_f = np.concatenate([[0], np.cumsum(req_f.new_len)])
    cand_full = np.concatenate([y_full[off_f[b + 1] - T:off_f[b + 1]] for b in range(3)])
    x_cand = to64(x_c)
    err = rel(y_c - x_cand, cand_full - x_cand)
    say(f"  candidates: cached vs full branch rel err {err:.2e}")
    assert err < TOL[full.dtype]
    req_f.close()
    req_c.close()


def test_layers_wide_model_bf16():
    """d_model 1024 against H*dh 256 (wider rows than the configurations'):
    the pre-norm statistics take four 512-value chunks a lane group."""
    say("wide model bf16 d=1024")
    cfg = small_config(dtype="bf16", d_model=1024, num_heads=2, head_dim=128, num_layers=2, n_targets=8,
                       cache="hit", page_size=32)
    hist = [90, 300]
    w = generate(cfg, 4, batch=len(hist), hist_override=hist)
    w.hit = np.ones(len(hist), bool)
    w.prefill_order = np.arange(len(hist), dtype=np.int32)
    w.num_pages = sum(-(-(h + 8) // 32) for h in hist) + 3
    w.page_perm = np.random.default_rng(5).permutation(w.num_pages).astype(np.int32)
    w.cfg = dataclasses.replace(cfg, batch=len(hist))
    for lw in w.layers:
        lw.w1 *= 4.0
        lw.w2 *= 4.0
    scn = runtime.Scenario(w)
    scn.prefill()
    req, x = scn.make_request()
    per = run_layers_with_taps(scn, req, x)
    worst = check_layers(scn, req, per, [0, 1], "wide")
    _assert_within(worst, TOL[scn.dtype])
    req.close()


def test_precomputed_w1_colsum_is_identical():
    """The layer with W1's column sums from hstu_w1_colsum and with the sums
    computed in the call give bit-identical outputs."""
    say("precomputed W1 column sums")
    w = _small("hit", "bf16", hist=[200, 33], T=16, layers=1)
    scn = runtime.Scenario(w)
    scn.prefill()
    req, x = scn.make_request()
    y1 = runtime.forward(scn.model, req, x, scn.cache).clone()
    saved = scn.model.w1_colsum
    scn.model.w1_colsum = [None] * len(saved)
    y2 = runtime.forward(scn.model, req, x, scn.cache).clone()   # appends the same K/V again
    scn.model.w1_colsum = saved
    torch.cuda.synchronize()
    assert saved[0] is not None and torch.equal(y1, y2)
    req.close()


def test_f2_row_statistics_slots():
    """f2's row statistics of y (mean and sum of squared deviations per
    128-column tile of the stored bf16 y) against float64 sums over the
    returned y, and the combined slots against one pass over the row."""
    from generative_recommender_sequence_amd import hstu
    say("f2 row statistics")
    w = _small("hit", "bf16", hist=[200, 33, 5], T=16, layers=1)
    scn = runtime.Scenario(w)
    scn.prefill()
    req, x = scn.make_request()
    model = scn.model
    n, d = x.shape
    slots = d // 128
    ws = runtime.workspace_for(model, req, x.device)
    y = torch.empty_like(x)
    stats = torch.full((n, slots, 2), float("nan"), dtype=torch.float32, device=x.device)
    a = runtime.layer_args(model, req, 0, x, y, scn.cache, ws)
    a.y_stats = stats.data_ptr()
    hstu.hstu_stack_forward([a], runtime.stream_handle())
    torch.cuda.synchronize()
    yt = to64(y).reshape(n, slots, 128)
    mean = yt.mean(axis=2)
    m2 = ((yt - mean[..., None]) ** 2).sum(axis=2)
    got = stats.cpu().numpy().astype(np.float64)
    e_mean = np.max(np.abs(got[..., 0] - mean)) / max(np.max(np.abs(yt)), 1e-30)
    e_m2 = np.max(np.abs(got[..., 1] - m2) / np.maximum(m2, 1e-30))
    say(f"  mean err {e_mean:.2e}  M2 rel err {e_m2:.2e}")
    assert e_mean < 1e-6 and e_m2 < 1e-5
    # the next layer's input statistics from slots equal those of one pass
    full_mean = yt.reshape(n, d).mean(axis=1)
    comb_mean = got[..., 0].mean(axis=1)
    comb_m2 = got[..., 1].sum(axis=1) + 128 * ((got[..., 0] - comb_mean[:, None]) ** 2).sum(axis=1)
    full_m2 = ((yt.reshape(n, d) - full_mean[:, None]) ** 2).sum(axis=1)
    assert np.max(np.abs(comb_m2 - full_m2) / full_m2) < 1e-5
    # a paged layer given x_stats must be given the rows' pool slots as well
    b = runtime.layer_args(model, req, 0, y, x.clone(), scn.cache, ws)
    b.x_stats = stats.data_ptr()
    with pytest.raises(RuntimeError, match="needs row_slots"):
        hstu.hstu_stack_forward([b], runtime.stream_handle())
    req.close()


def test_row_statistics_need_narrow_bf16():
    """x_stats / y_stats are refused for d_model above 512."""
    from generative_recommender_sequence_amd import hstu
    cfg = small_config(dtype="bf16", d_model=1024, num_heads=2, head_dim=128, num_layers=1, n_targets=8)
    w = generate(cfg, 4, batch=2, hist_override=[40, 20])
    scn = runtime.Scenario(w)
    req, x = scn.make_request()
    ws = runtime.workspace_for(scn.model, req, x.device)
    y = torch.empty_like(x)
    stats = torch.empty((x.shape[0], 8, 2), dtype=torch.float32, device=x.device)
    a = runtime.layer_args(scn.model, req, 0, x, y, None, ws)
    a.y_stats = stats.data_ptr()
    with pytest.raises(RuntimeError, match="d_model <= 512"):
        hstu.hstu_stack_forward([a], runtime.stream_handle())
    req.close()


def test_empty_request_is_a_no_op():
    """A request whose users bring no new tokens: attention returns no rows,
    and the stack returns an empty output and leaves the cache as it was."""
    from generative_recommender_sequence_amd import hstu
    say("empty request")
    w = _small("hit", "bf16", hist=[200, 33], T=16, layers=2)
    scn = runtime.Scenario(w)
    scn.prefill()
    users = scn.request_inputs()[0]
    before = hstu.kv_lookup(scn.cache.h, users).copy()
    free_before = hstu.kv_free_pages(scn.cache.h)
    req = runtime.prepare(scn.cache, users, [0, 0], [0, 0], [1.0, 1.0], scn.max_pages, scn.cfg.num_heads,
                          scn.cfg.head_dim)
    assert int(req.info.n_new_total) == 0
    x = torch.empty((0, scn.cfg.d_model), dtype=torch.bfloat16, device="cuda")
    y = runtime.forward(scn.model, req, x, scn.cache)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, scn.cfg.d_model)
    assert np.array_equal(hstu.kv_lookup(scn.cache.h, users), before)
    assert hstu.kv_free_pages(scn.cache.h) == free_before
    req.close()
    # attention alone over a contiguous prefix, with no queries
    H, dh = scn.cfg.num_heads, scn.cfg.head_dim
    areq = runtime.prepare_attn(None, [0, 1], [0, 0], [0, 0], [1.0, 1.0], 0, H, dh, cached_len=[5, 0])
    kv = torch.zeros((5, H * dh), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((0, H * dh), dtype=torch.bfloat16, device="cuda")
    o = runtime.attention(areq, q, H * dh, scn.model.rab[0], hstu.HSTU_BF16, kv, kv, H * dh)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (0, H * dh)
    areq.close()


@pytest.mark.parametrize("seed", range(3))
def test_layers_random_hit_and_miss_bf16(seed):
    """Seeded random batches through two cached layers: 1-5 users with random
    history lengths, candidate counts and hit/miss flags, page size 32 or 64."""
    rng = np.random.default_rng(2000 + seed)
    B = int(rng.integers(1, 6))
    hist = [int(h) for h in rng.integers(1, 700, size=B)]
    T = int(rng.integers(1, 65))
    hit = [bool(b) for b in rng.integers(0, 2, size=B)]
    P = int(rng.choice([32, 64]))
    say(f"random layers seed={seed} hist={hist} T={T} hit={hit} P={P}")
    w = _small("hit", "bf16", hist=hist, T=T, P=P, hit=hit, seed=seed)
    scn = runtime.Scenario(w)
    scn.prefill()
    req, x = scn.make_request()
    per = run_layers_with_taps(scn, req, x)
    worst = check_layers(scn, req, per, list(range(B)), f"random-{seed}")
    _assert_within(worst, TOL[scn.dtype])
    req.close()


def _edge_rows(rng, n, d, kind):
    """Layer-input rows that stress a LayerNorm: a large mean against the
    spread, constant rows with a few elements off by a few units in the last
    place, or variances of the order of eps; all bf16-exact."""
    if kind == "large_mean":
        m = rng.choice([-300.0, -30.0, 30.0, 100.0, 300.0], size=(n, 1))
        return round_bf16((m + rng.standard_normal((n, d))).astype(np.float32))
    if kind == "constant_but_few":
        x = np.full((n, d), 1000.0, np.float32)
        for r in range(n):
            idx = rng.choice(d, size=4, replace=False)
            x[r, idx] += rng.choice([-16.0, -8.0, 8.0, 16.0], size=4)
        return round_bf16(x)
    if kind == "near_eps":
        sd = np.sqrt(rng.choice([1e-6, 1e-5, 1e-4], size=(n, 1)))
        return round_bf16((sd * rng.standard_normal((n, d))).astype(np.float32))
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["large_mean", "constant_but_few", "near_eps"])
def test_prenorm_edge_rows_bf16(kind):
    """The bf16 pre-norm is folded into f1 as rstd (x . W1 - mean colsum(W1))
    on the raw rows, and later layers take row statistics f2 computed from
    per-tile pieces: rows whose mean dwarfs their spread, or whose variance
    is of the order of eps, go through both (two layers, cached and
    recomputed users, the cache pre-filled from the same kind of rows)."""
    say(f"pre-norm edge rows: {kind}")
    w = _small("hit", "bf16", hist=[150, 300, 90], T=16, hit=[True, False, True], seed=11)
    rng = np.random.default_rng(77)
    d = w.cfg.d_model
    w.x = [_edge_rows(rng, len(xb), d, kind) for xb in w.x]
    scn = runtime.Scenario(w)
    scn.prefill()
    req, x = scn.make_request()
    per = run_layers_with_taps(scn, req, x)
    worst = check_layers(scn, req, per, [0, 1, 2], f"prenorm-{kind}")
    _assert_within(worst, TOL[scn.dtype])
    req.close()


@pytest.mark.parametrize("kind", ["o_large_mean", "o_near_eps"])
def test_attention_output_layernorm_edge_bf16(kind):
    """LayerNorm(o) on attention outputs whose H*dh values share a large mean
    against their spread (W1's V columns nearly equal, so every value column
    of V is nearly the same), or whose variance is below eps (V scaled down a
    thousandfold)."""
    say(f"LN(o) edge: {kind}")
    w = _small("hit", "bf16", hist=[200, 700, 60], T=16, hit=[True, False, True], seed=12)
    rng = np.random.default_rng(78)
    inner = w.cfg.inner
    for lw in w.layers:
        wv = lw.w1[:, inner:2 * inner]
        if kind == "o_large_mean":
            base = np.abs(wv[:, :1]) + 0.05
            lw.w1[:, inner:2 * inner] = round_bf16((base * (1.0 + 0.05 * rng.standard_normal(wv.shape))).astype(
                np.float32))
        else:
            lw.w1[:, inner:2 * inner] = round_bf16((wv * 1e-3).astype(np.float32))
    scn = runtime.Scenario(w)
    scn.prefill()
    req, x = scn.make_request()
    per = run_layers_with_taps(scn, req, x)
    o = to64(per[0]["o"])
    mu, sd = o.mean(axis=1), o.std(axis=1)
    say(f"  o rows: median |mean|/std {np.median(np.abs(mu) / np.maximum(sd, 1e-30)):.1f}, "
        f"median variance {np.median(sd ** 2):.2e}")
    worst = check_layers(scn, req, per, [0, 1, 2], f"ln-o-{kind}")
    _assert_within(worst, TOL[scn.dtype])
    req.close()


def test_layer_longest_cached_user_wide_model_bf16():
    """The row that sums the most partial tiles: one user at the longest
    supported sequence (65,471 cached positions + 64 candidates = 65,535) in
    16-token pages, d_model 1024, one layer.  Each candidate row's output is
    the key-order sum of several hundred pieces' fp32 partial tiles; the
    layer (through LN(o), the gate and f2) must stay within the bound."""
    say("longest cached user, wide model bf16")
    hist = [65471]
    cfg = small_config(dtype="bf16", d_model=1024, num_heads=2, head_dim=128, num_layers=1, n_targets=64,
                       cache="hit", page_size=16)
    w = generate(cfg, 8, batch=1, hist_override=hist)
    w.hit = np.ones(1, bool)
    w.prefill_order = np.arange(1, dtype=np.int32)
    w.num_pages = -(-(hist[0] + 64) // 16) + 3
    w.page_perm = np.random.default_rng(9).permutation(w.num_pages).astype(np.int32)
    w.cfg = dataclasses.replace(cfg, batch=1)
    scn = runtime.Scenario(w)
    scn.prefill()
    req, x = scn.make_request()
    items = hstu.hstu_plan_get_items(req.plan)
    pieces = int((items[:, 5] >= 0).sum())
    per = run_layers_with_taps(scn, req, x)
    worst = check_layers(scn, req, per, [0], "longest")
    say(f"  {pieces} pieces over 2 heads")
    assert pieces >= 64
    _assert_within(worst, TOL[scn.dtype])
    req.close()

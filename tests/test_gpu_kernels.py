"""GPU parity of the individual C-ABI calls: kv_page_append / kv_page_gather
(byte-exact against the oracle's pool-placement model) and hstu_attn_fwd
(against the oracle attention) in fp32 and bf16, contiguous and paged,
across ragged lengths that span several 64-key tiles and 128-query blocks."""
import numpy as np
import pytest
import torch

import oracle
from generative_recommender_sequence_amd import hstu, runtime
from generative_recommender_sequence_amd.hstu import HSTU_BF16, HSTU_F32
from generative_recommender_sequence_amd.workloads import round_bf16
from gpu_checks import TOL, rel, say, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    runtime.require_gpu()


def _bits_tensor(rng, shape, dtype):
    if dtype == HSTU_BF16:
        b = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        return b, torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)
    b = rng.integers(0, 1 << 32, size=shape, dtype=np.uint32)
    return b, torch.from_numpy(b.view(np.int32)).cuda().view(torch.float32)


def _pool_bits(t: torch.Tensor, dtype):
    if dtype == HSTU_BF16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("dtype,P,dh", [(HSTU_BF16, 32, 128), (HSTU_BF16, 64, 128), (HSTU_F32, 32, 32),
                                        (HSTU_F32, 16, 64)])
def test_append_then_gather_is_byte_exact(dtype, P, dh):
    say(f"append/gather dtype={dtype} P={P} dh={dh}")
    rng = np.random.default_rng(P + dh)
    H, layers = 2, 3
    users = [10, 11, 12, 13, 14, 15]
    hist = [0, 37, 64, 1, 130, 0]
    new = [5, 27, 0, 64, 3, 0]
    inner = H * dh
    num_pages = sum(-(-(h + t) // P) for h, t in zip(hist, new)) + 3
    perm = rng.permutation(num_pages)
    cache = runtime.PagedCache(layers, H, dh, P, num_pages, dtype, perm)
    expect = np.zeros(layers * num_pages * H * P * dh, np.uint16 if dtype == HSTU_BF16 else np.uint32)
    expect_v = expect.copy()
    expect[:] = _pool_bits(cache.k_pool, dtype)
    expect_v[:] = _pool_bits(cache.v_pool, dtype)
    max_pages = 16
    rows_k, rows_v = {}, {}
    s = runtime.stream_handle()
    for phase, counts in enumerate((hist, new)):
        pt, kl = hstu.kv_page_alloc(cache.h, users, counts, max_pages)
        start = (kl - np.asarray(counts)).astype(np.int32)
        off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        n = int(off[-1])
        stride = 4 * inner                       # rows embedded in a wider buffer
        kb, kt = _bits_tensor(rng, (max(n, 1), stride), dtype)
        vb, vt = _bits_tensor(rng, (max(n, 1), stride), dtype)
        d_off = torch.from_numpy(off).cuda()
        d_start = torch.from_numpy(start).cuda()
        d_pt = torch.from_numpy(pt).cuda()
        layer = 1 + phase
        hstu.kv_page_append(cache.h, layer, len(users), d_off.data_ptr(), d_start.data_ptr(), d_pt.data_ptr(),
                            max_pages, kt.data_ptr() + inner * (2 if dtype == HSTU_BF16 else 4),
                            vt.data_ptr(), stride, n, s)
        for b in range(len(users)):
            rk = kb[off[b]:off[b + 1], inner:2 * inner]
            rv = vb[off[b]:off[b + 1], :inner]
            oracle.pool_place(expect, layer, pt[b], int(start[b]), rk, num_pages, H, P, dh)
            oracle.pool_place(expect_v, layer, pt[b], int(start[b]), rv, num_pages, H, P, dh)
            rows_k[(layer, b)], rows_v[(layer, b)] = rk, rv
    torch.cuda.synchronize()
    assert np.array_equal(_pool_bits(cache.k_pool, dtype), expect)
    assert np.array_equal(_pool_bits(cache.v_pool, dtype), expect_v)
    # gather layer 1 (histories) back out
    pt, kl = hstu.kv_page_table(cache.h, users, max_pages)
    lens = np.asarray(hist, np.int32)
    out_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = int(out_off[-1])
    t = runtime.tdtype(dtype)
    ko = torch.zeros((n, inner), dtype=t, device="cuda")
    vo = torch.zeros((n, inner), dtype=t, device="cuda")
    d_pt, d_len, d_off = (torch.from_numpy(a).cuda() for a in (pt, lens, out_off))
    hstu.kv_page_gather(cache.h, 1, len(users), d_pt.data_ptr(), max_pages, d_len.data_ptr(), d_off.data_ptr(),
                        n, ko.data_ptr(), vo.data_ptr(), s)
    torch.cuda.synchronize()
    want_k = np.concatenate([rows_k[(1, b)] for b in range(len(users))])
    want_v = np.concatenate([rows_v[(1, b)] for b in range(len(users))])
    assert np.array_equal(_pool_bits(ko, dtype).reshape(n, inner), want_k)
    assert np.array_equal(_pool_bits(vo, dtype).reshape(n, inner), want_v)


def _attn_case(rng, dtype, H, dh, new_len, cached_len, n_targets, scale=0.5):
    L = [c + t for c, t in zip(cached_len, new_len)]
    rnd = round_bf16 if dtype == HSTU_BF16 else (lambda a: a.astype(np.float32))
    q = rnd((rng.standard_normal((sum(new_len), H * dh)) * scale).astype(np.float32))
    k = rnd((rng.standard_normal((sum(L), H * dh)) * scale).astype(np.float32))
    v = rnd(rng.standard_normal((sum(L), H * dh)).astype(np.float32))
    rab = rnd((rng.standard_normal(64) * 0.5).astype(np.float32))
    return q, k, v, rab, L


ATTN_CASES = [
    # new_len, cached_len, n_targets
    ([37, 64], [0, 0], [0, 0]),                               # the tiny causal case
    ([1, 129, 300, 0, 65], [0, 0, 0, 0, 0], [0, 64, 17, 0, 1]),  # ragged, candidates, an empty user
    ([64, 256, 3], [700, 1500, 0], [64, 256, 3]),              # cached prefixes + candidate blocks
    ([520], [3000], [7]),                                      # history queries after a cache
]


@pytest.mark.parametrize("dtype,dh", [(HSTU_F32, 32), (HSTU_F32, 64), (HSTU_F32, 128), (HSTU_BF16, 128)])
@pytest.mark.parametrize("case", range(len(ATTN_CASES)))
def test_attention_contiguous_vs_oracle(dtype, dh, case):
    new_len, cached_len, n_targets = ATTN_CASES[case]
    say(f"attention contiguous dtype={dtype} dh={dh} case={case}")
    rng = np.random.default_rng(case * 7 + dh)
    H = 2
    q, k, v, rab, L = _attn_case(rng, dtype, H, dh, new_len, cached_len, n_targets)
    norm_n = [float(x) + 0.5 for x in L]
    ref = oracle.attention(q, k, v, new_len, cached_len, L, n_targets, norm_n, rab, H, dh)
    t = runtime.tdtype(dtype)
    req = runtime.prepare_attn(None, list(range(len(new_len))), new_len, n_targets, norm_n, 0, H, dh,
                               cached_len=cached_len)
    qd, kd, vd = (torch.from_numpy(a).to("cuda", t) for a in (q, k, v))
    rabd = torch.from_numpy(rab).cuda()
    o = runtime.attention(req, qd, H * dh, rabd, dtype, kd, vd, H * dh)
    torch.cuda.synchronize()
    err = rel(to64(o), ref)
    say(f"  rel err {err:.2e}")
    assert err < TOL[dtype]
    req.close()


def _paged_setup(rng, dtype, H, dh, P, new_len, cached_len, n_targets, free_order_seed):
    q, k, v, rab, L = _attn_case(rng, dtype, H, dh, new_len, cached_len, n_targets)
    users = [100 + i for i in range(len(new_len))]
    num_pages = sum(-(-l // P) for l in L) + 2
    perm = np.random.default_rng(free_order_seed).permutation(num_pages)
    cache = runtime.PagedCache(1, H, dh, P, num_pages, dtype, perm)
    max_pages = max(-(-l // P) for l in L)
    pt, kl = hstu.kv_page_alloc(cache.h, users, L, max_pages)
    off = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    t = runtime.tdtype(dtype)
    kd, vd = (torch.from_numpy(a).to("cuda", t) for a in (k, v))
    d_off = torch.from_numpy(off).cuda()
    d_start = torch.zeros(len(L), dtype=torch.int32, device="cuda")
    d_pt = torch.from_numpy(pt).cuda()
    hstu.kv_page_append(cache.h, 0, len(L), d_off.data_ptr(), d_start.data_ptr(), d_pt.data_ptr(), max_pages,
                        kd.data_ptr(), vd.data_ptr(), H * dh, int(off[-1]), runtime.stream_handle())
    return q, k, v, rab, L, users, cache, max_pages


@pytest.mark.parametrize("dtype,dh,P", [(HSTU_F32, 64, 16), (HSTU_BF16, 128, 32), (HSTU_BF16, 128, 64)])
@pytest.mark.parametrize("case", [1, 2, 3])
def test_attention_paged_vs_oracle(dtype, dh, P, case):
    new_len, cached_len, n_targets = ATTN_CASES[case]
    say(f"attention paged dtype={dtype} dh={dh} P={P} case={case}")
    rng = np.random.default_rng(case * 11 + P)
    H = 2
    q, k, v, rab, L, users, cache, max_pages = _paged_setup(rng, dtype, H, dh, P, new_len, cached_len,
                                                            n_targets, 5)
    norm_n = [float(x) for x in L]
    ref = oracle.attention(q, k, v, new_len, cached_len, L, n_targets, norm_n, rab, H, dh)
    req = runtime.prepare_attn(cache, users, new_len, n_targets, norm_n, max_pages, H, dh)
    qd = torch.from_numpy(q).to("cuda", runtime.tdtype(dtype))
    o = runtime.attention(req, qd, H * dh, torch.from_numpy(rab).cuda(), dtype, cache=cache)
    torch.cuda.synchronize()
    err = rel(to64(o), ref)
    say(f"  rel err {err:.2e}")
    assert err < TOL[dtype]
    req.close()


def test_attention_page_placement_and_size_invariance():
    """Reduction order depends only on logical positions: a different physical
    page placement gives byte-identical output; a different page size too."""
    say("attention page placement / size invariance")
    new_len, cached_len, n_targets = ATTN_CASES[2]
    outs = []
    for P, seed in ((32, 1), (32, 2), (64, 3)):
        rng = np.random.default_rng(42)
        q, k, v, rab, L, users, cache, max_pages = _paged_setup(rng, HSTU_BF16, 2, 128, P, new_len,
                                                                cached_len, n_targets, seed)
        req = runtime.prepare_attn(cache, users, new_len, n_targets, None, max_pages, 2, 128)
        qd = torch.from_numpy(q).to("cuda", torch.bfloat16)
        outs.append(runtime.attention(req, qd, 256, torch.from_numpy(rab).cuda(), HSTU_BF16, cache=cache))
        torch.cuda.synchronize()
        req.close()
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("paged", [False, True])
def test_attention_at_maximum_length(paged):
    """One user at the longest sequence a plan accepts (65,535 positions: a
    65,471-token history and 64 candidates), bf16: distances up to 65,534
    fall in the last rab bucket, and the paged user spans 1,024 pages."""
    new_len, cached_len, n_targets = [64], [65471], [64]
    say(f"attention at maximum length paged={paged}")
    rng = np.random.default_rng(17)
    H, dh, dtype = 2, 128, HSTU_BF16
    t = runtime.tdtype(dtype)
    if paged:
        q, k, v, rab, L, users, cache, max_pages = _paged_setup(rng, dtype, H, dh, 64, new_len, cached_len,
                                                                n_targets, 3)
        norm_n = [float(x) for x in L]
        req = runtime.prepare_attn(cache, users, new_len, n_targets, norm_n, max_pages, H, dh)
        o = runtime.attention(req, torch.from_numpy(q).to("cuda", t), H * dh, torch.from_numpy(rab).cuda(), dtype,
                              cache=cache)
    else:
        q, k, v, rab, L = _attn_case(rng, dtype, H, dh, new_len, cached_len, n_targets)
        norm_n = [float(x) for x in L]
        req = runtime.prepare_attn(None, [0], new_len, n_targets, norm_n, 0, H, dh, cached_len=cached_len)
        qd, kd, vd = (torch.from_numpy(a).to("cuda", t) for a in (q, k, v))
        o = runtime.attention(req, qd, H * dh, torch.from_numpy(rab).cuda(), dtype, kd, vd, H * dh)
    torch.cuda.synchronize()
    assert L == [65535]
    ref = oracle.attention(q, k, v, new_len, cached_len, L, n_targets, norm_n, rab, H, dh)
    err = rel(to64(o), ref)
    say(f"  rel err {err:.2e}")
    assert err < TOL[dtype]
    req.close()


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("paged", [False, True])
def test_attention_random_jagged_batches(seed, paged):
    """Seeded random batches (1-6 users, up to 900 positions each, a random
    cached/new split and candidate count), bf16: the plan's splitting of each
    (q-block, head) into pieces and the key-order sum of their partial tiles
    on shapes no fixed case picks."""
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 7))
    L = rng.integers(1, 901, size=B)
    new_len = [int(rng.integers(0, l + 1)) for l in L]
    cached_len = [int(l) - t for l, t in zip(L, new_len)]
    n_targets = [int(rng.integers(0, t + 1)) if t else 0 for t in new_len]
    say(f"attention random seed={seed} paged={paged} L={list(map(int, L))} new={new_len} T={n_targets}")
    H, dh, dtype = 2, 128, HSTU_BF16
    t = runtime.tdtype(dtype)
    if paged:
        q, k, v, rab, Ls, users, cache, max_pages = _paged_setup(rng, dtype, H, dh, 32, new_len, cached_len,
                                                                 n_targets, seed)
        norm_n = [float(x) for x in Ls]
        req = runtime.prepare_attn(cache, users, new_len, n_targets, norm_n, max_pages, H, dh)
        o = runtime.attention(req, torch.from_numpy(q).to("cuda", t), H * dh, torch.from_numpy(rab).cuda(), dtype,
                              cache=cache)
    else:
        q, k, v, rab, Ls = _attn_case(rng, dtype, H, dh, new_len, cached_len, n_targets)
        norm_n = [float(x) for x in Ls]
        req = runtime.prepare_attn(None, list(range(B)), new_len, n_targets, norm_n, 0, H, dh,
                                   cached_len=cached_len)
        qd, kd, vd = (torch.from_numpy(a).to("cuda", t) for a in (q, k, v))
        o = runtime.attention(req, qd, H * dh, torch.from_numpy(rab).cuda(), dtype, kd, vd, H * dh)
    torch.cuda.synchronize()
    ref = oracle.attention(q, k, v, new_len, cached_len, Ls, n_targets, norm_n, rab, H, dh)
    if ref.size:
        err = rel(to64(o), ref)
        say(f"  rel err {err:.2e}")
        assert err < TOL[dtype]
    else:
        assert o.numel() == 0
    req.close()


@pytest.mark.parametrize("case", [([40000], [100], [40000]), ([30000], [3000], [30000])])
def test_attention_candidates_far_past_a_short_history(case):
    """16-token pages, a short cached history and tens of thousands of
    candidates: a candidate block sees the history's first tiles and its own
    diagonal tiles thousands of positions later, so the plan must cut its
    pieces for each to stage at most 2048 page-table entries."""
    new_len, cached_len, n_targets = case
    say(f"attention far candidates new={new_len} cached={cached_len} P=16")
    rng = np.random.default_rng(23)
    H, dh, dtype, P = 2, 128, HSTU_BF16, 16
    q, k, v, rab, L, users, cache, max_pages = _paged_setup(rng, dtype, H, dh, P, new_len, cached_len,
                                                            n_targets, 9)
    norm_n = [float(x) for x in L]
    req = runtime.prepare_attn(cache, users, new_len, n_targets, norm_n, max_pages, H, dh)
    items = hstu.hstu_plan_get_items(req.plan)
    real = items[items[:, 5] >= 0]
    span = -(-(real[:, 4] * 64) // P) - (real[:, 3] * 64) // P
    assert span.max() <= 2048
    o = runtime.attention(req, torch.from_numpy(q).to("cuda", runtime.tdtype(dtype)), H * dh,
                          torch.from_numpy(rab).cuda(), dtype, cache=cache)
    torch.cuda.synchronize()
    ref = oracle.attention(q, k, v, new_len, cached_len, L, n_targets, norm_n, rab, H, dh)
    err = rel(to64(o), ref)
    say(f"  rel err {err:.2e} (largest item span {int(span.max())} pages)")
    assert err < TOL[dtype]
    req.close()


def test_attention_split_timing_launch_is_identical():
    """The instrumented launch that runs users with a cached prefix and users
    without one as two grids gives byte-identical output to the single grid,
    and records both parts."""
    new_len, cached_len, n_targets = [64, 700, 64, 300], [1500, 0, 900, 0], [64, 64, 64, 17]
    say("attention split timing launch")
    rng = np.random.default_rng(31)
    H, dh, dtype = 2, 128, HSTU_BF16
    q, k, v, rab, L, users, cache, max_pages = _paged_setup(rng, dtype, H, dh, 32, new_len, cached_len,
                                                            n_targets, 4)
    # the two orders are part of plans made while split timing is on
    hstu.hstu_timing_enable(True, split_attention=True)
    req = runtime.prepare_attn(cache, users, new_len, n_targets, None, max_pages, H, dh)
    hstu.hstu_timing_enable(False)
    qd = torch.from_numpy(q).to("cuda", torch.bfloat16)
    rabd = torch.from_numpy(rab).cuda()
    o1 = runtime.attention(req, qd, H * dh, rabd, dtype, cache=cache)
    hstu.hstu_timing_enable(True, split_attention=True)
    o2 = runtime.attention(req, qd, H * dh, rabd, dtype, cache=cache)
    torch.cuda.synchronize()
    n_c, _ = hstu.hstu_timing_read("attention_cached")
    n_p, _ = hstu.hstu_timing_read("attention_prefill")
    n_a, _ = hstu.hstu_timing_read("attention")
    hstu.hstu_timing_enable(False)
    assert (n_c, n_p, n_a) == (1, 1, 0)
    assert torch.equal(o1, o2)
    req.close()


def test_attention_phase_records():
    """With a phase-record buffer registered, every block of the bf16
    attention writes its record (ordered stamps, its work item's slot and
    tile range) and the output is byte-identical to a launch without one."""
    new_len, cached_len, n_targets = [64, 700, 64, 300], [1500, 0, 900, 0], [64, 64, 64, 17]
    say("attention phase records")
    rng = np.random.default_rng(37)
    H, dh, dtype = 2, 128, HSTU_BF16
    q, k, v, rab, L, users, cache, max_pages = _paged_setup(rng, dtype, H, dh, 32, new_len, cached_len,
                                                            n_targets, 4)
    req = runtime.prepare_attn(cache, users, new_len, n_targets, None, max_pages, H, dh)
    items = hstu.hstu_plan_get_items(req.plan)
    qd = torch.from_numpy(q).to("cuda", torch.bfloat16)
    rabd = torch.from_numpy(rab).cuda()
    o1 = runtime.attention(req, qd, H * dh, rabd, dtype, cache=cache)
    n = len(items)
    rec = hstu.ATTN_STAMP_DTYPE.itemsize
    buf = torch.zeros(n * rec // 8, dtype=torch.int64, device="cuda")
    hstu.hstu_attn_stamps(buf.data_ptr(), n)
    try:
        o2 = runtime.attention(req, qd, H * dh, rabd, dtype, cache=cache)
        torch.cuda.synchronize()
    finally:
        hstu.hstu_attn_stamps(0, 0)
    a = np.frombuffer(buf.cpu().numpy().tobytes(), dtype=hstu.ATTN_STAMP_DTYPE)
    real = items[:, 5] >= 0
    assert torch.equal(o1, o2)
    assert (a["end"][~real] == 0).all()
    r = a[real]
    assert (r["start"] > 0).all()
    assert (r["start"] <= r["setup_done"]).all() and (r["setup_done"] <= r["loop_done"]).all()
    assert (r["loop_done"] <= r["end"]).all()
    np.testing.assert_array_equal(r["slot"], items[real, 5])
    np.testing.assert_array_equal(r["tiles"], items[real, 4] - items[real, 3])
    assert (r["xcc_id"] < 8).all()
    # a record buffer smaller than the plan is not used
    small = torch.zeros(8, dtype=torch.int64, device="cuda")
    hstu.hstu_attn_stamps(small.data_ptr(), 1)
    try:
        o3 = runtime.attention(req, qd, H * dh, rabd, dtype, cache=cache)
        torch.cuda.synchronize()
    finally:
        hstu.hstu_attn_stamps(0, 0)
    assert torch.equal(o1, o3) and int(small.abs().sum()) == 0
    req.close()

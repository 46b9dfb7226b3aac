"""GPU parity at the five workload configurations' full sizes, in the launch
configuration the benchmark times: every layer of sampled users is checked
against the oracle (fed the GPU's layer input and cache bytes); the cache
metadata after pre-fill, lookup, eviction and allocation is compared byte for
byte with the oracle allocator; cached candidates are compared with a full
recompute of the same data."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from generative_recommender_sequence_amd import hstu, runtime
from generative_recommender_sequence_amd.workloads import workload_for
from gpu_checks import TOL, check_layers, rel, run_layers_with_taps, say, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    runtime.require_gpu()


def _sample(w, k=2):
    """indices of the shortest users (the oracle runs them in seconds) and,
    when cached, at least one cached user"""
    L = w.hist_len + w.n_targets
    order = list(np.argsort(L, kind="stable"))
    pick = order[:k]
    if w.cfg.cache == "mixed":
        hits = [b for b in order if w.hit[b]][:1]
        miss = [b for b in order if not w.hit[b]][:1]
        pick = hits + miss
    return sorted(int(b) for b in pick)


def _oracle_cache_ops(scn):
    """Replays the scenario's host cache operations on the oracle allocator."""
    w, cfg = scn.w, scn.cfg
    ko = oracle.KVOracle(w.num_pages, cfg.page_size, w.page_perm)
    cached_users = [(w.user_ids[b], int(w.hist_len[b])) for b in range(cfg.batch) if w.hit[b]]
    cached_users += [(w.stale_ids[s], int(w.stale_hist_len[s])) for s in range(len(w.stale_ids))]
    order = [cached_users[i] for i in w.prefill_order]
    if order:
        rc, _, _ = ko.alloc([u for u, _ in order], [n for _, n in order], scn.max_pages)
        assert rc == 0
    return ko


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_config_parity(name):
    say(f"config {name}")
    w = workload_for(name, 0)
    scn = runtime.Scenario(w)
    scn.prefill()
    if scn.cache is not None:
        ko = _oracle_cache_ops(scn)
        assert hstu.kv_state_dump(scn.cache.h) == ko.dump(), "pre-fill state differs from the oracle"
    req, x = scn.make_request()
    if scn.cache is not None:
        users, new_len, _, _, _ = scn.request_inputs()
        rc, cached = ko.lookup(users)
        need = scn.cache.pages_needed(cached, new_len)
        rc, ev = ko.evict_lru(need, users)
        assert rc == 0 and list(ev) == list(req.evicted)
        rc, pt, kl = ko.alloc(users, new_len, scn.max_pages)
        assert rc == 0
        assert np.array_equal(pt, req.page_table.cpu().numpy()) and np.array_equal(kl, req.kv_len)
        assert hstu.kv_state_dump(scn.cache.h) == ko.dump(), "request state differs from the oracle"
        if w.cfg.cache == "mixed":
            assert len(req.evicted) > 0, "the pool must force an eviction"
    per = run_layers_with_taps(scn, req, x)
    sample = _sample(w) if name != "C1" else [0, 1]
    worst = check_layers(scn, req, per, sample, name)
    tol = TOL[scn.dtype]
    bad = {k: v for k, v in worst.items() if not v < tol}
    assert not bad, f"{name} over tolerance {tol}: {bad}"
    req.close()


def test_c3_candidates_match_c2_full_recompute():
    say("C3 (cached) vs C2 (full recompute)")
    w3 = workload_for("C3", 0)
    w2 = dataclasses.replace(w3, cfg=dataclasses.replace(w3.cfg, cache="none"),
                             hit=np.zeros(w3.cfg.batch, bool))
    s2 = runtime.Scenario(w2)
    r2, x2 = s2.make_request()
    y2 = to64(runtime.forward(s2.model, r2, x2, None))
    s3 = runtime.Scenario(w3)
    s3.prefill()
    r3, x3 = s3.make_request()
    y3 = to64(runtime.forward(s3.model, r3, x3, s3.cache))
    torch.cuda.synchronize()
    off = np.concatenate([[0], np.cumsum(r2.new_len)])
    T = w3.cfg.n_targets
    cand = np.concatenate([y2[off[b + 1] - T:off[b + 1]] for b in range(w3.cfg.batch)])
    xc = to64(x3)
    err_y = rel(y3, cand)
    err_b = rel(y3 - xc, cand - xc)
    say(f"  Y rel {err_y:.2e}, branch rel {err_b:.2e}")
    assert err_y < 2e-2
    assert err_b < 5e-2
    r2.close()
    r3.close()

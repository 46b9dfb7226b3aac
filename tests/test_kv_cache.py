"""Cache metadata: the pure-Python model, the oracle allocator and the
library's manager must agree byte for byte on seeded operation sequences,
including pool exhaustion and the all-pinned case (host only, no GPU)."""
import numpy as np
import pytest

import oracle
from kv_model import (ERR_INVALID, ERR_NO_SPACE, ERR_UNKNOWN_USER, OK, KVModel, random_ops)


def _apply(impl, op):
    kind = op[0]
    if kind == "lookup":
        rc, lens = impl.lookup(op[1])
        return (rc, None if rc else [int(x) for x in lens])
    if kind == "alloc":
        rc, table, lens = impl.alloc(op[1], op[2], op[3])
        if rc:
            return (rc,)
        return (rc, [[int(p) for p in row] for row in table], [int(x) for x in lens])
    if kind == "evict":
        rc, ev = impl.evict_lru(op[1], op[2])
        return (rc, [int(e) for e in ev])
    if kind == "truncate":
        return (impl.truncate(op[1], op[2]),)
    if kind == "victims":
        rc, ev = impl.lru_victims(op[1], op[2])
        return (rc, [int(e) for e in ev])
    if kind == "offload":
        rc, dropped = impl.offload(op[1], op[2])
        return (rc, [int(d) for d in dropped])
    if kind == "onboard":
        return (impl.onboard(op[1]),)
    if kind == "residency":
        rc, where, lens = impl.residency(op[1])
        return (rc, [int(w) for w in where], [int(x) for x in lens])
    raise ValueError(kind)


def _impls(num_pages, page_size, free_order, with_lib=False):
    impls = {"model": KVModel(num_pages, page_size, free_order),
             "oracle": oracle.KVOracle(num_pages, page_size, free_order)}
    if with_lib:
        from generative_recommender_sequence_amd import hstu
        impls["lib"] = hstu.KVCache.host_only(num_pages, page_size, free_order)
    return impls


def _run_sequence(seed, with_lib=False, host_tier=False):
    rng = np.random.default_rng(seed)
    num_pages = int(rng.integers(4, 40))
    page_size = int(rng.choice([1, 2, 4, 32]))
    free_order = rng.permutation(num_pages)
    impls = _impls(num_pages, page_size, free_order, with_lib)
    if host_tier:
        host_pages = int(rng.integers(0, 30))
        for impl in impls.values():
            assert impl.host_attach(host_pages) == OK
            assert impl.host_attach(host_pages) == ERR_INVALID     # once per cache
    for op in random_ops(rng, 80 if host_tier else 60, max_new=3 * page_size + 2, host_tier=host_tier):
        results = {name: _apply(impl, op) for name, impl in impls.items()}
        first = results["model"]
        for name, r in results.items():
            assert r == first, f"seed {seed} op {op}: {name} {r} != model {first}"
        dumps = {name: impl.dump() for name, impl in impls.items()}
        for name, dmp in dumps.items():
            assert dmp == dumps["model"], f"seed {seed} op {op}: {name} dump differs"
        impls["model"].check_invariants()


@pytest.mark.parametrize("seed", range(40))
def test_model_vs_oracle_allocator(seed):
    _run_sequence(seed)


@pytest.mark.parametrize("seed", range(40, 100))
def test_library_vs_model_vs_oracle(seed):
    _run_sequence(seed, with_lib=True)


@pytest.mark.parametrize("seed", range(100, 140))
def test_host_tier_library_vs_model_vs_oracle(seed):
    _run_sequence(seed, with_lib=True, host_tier=True)


def test_host_tier_rules():
    for impl in _impls(6, 2, None, with_lib=True).values():
        assert impl.offload([1])[0] == ERR_INVALID                # no host tier yet
        assert impl.host_attach(5) == OK
        assert impl.alloc([1, 2], [3, 4], 4)[0] == OK             # 1: pages 0 1, 2: pages 2 3
        assert impl.lookup([2])[0] == OK                          # tick(2) > tick(1)
        rc, dropped = impl.offload([2, 1])
        assert rc == OK and len(dropped) == 0
        rc, where, lens = impl.residency([1, 2, 3])
        assert rc == OK and list(where) == [2, 2, 0] and list(lens) == [3, 4, 0]
        rc, lens = impl.lookup([1, 2])
        assert rc == OK and [int(x) for x in lens] == [0, 0]      # host users count as absent
        assert impl.alloc([1], [1], 4)[0] == ERR_INVALID          # not while on the host tier
        assert impl.truncate(1, 0) == ERR_UNKNOWN_USER
        assert impl.offload([3])[0] == ERR_UNKNOWN_USER
        assert impl.onboard([3]) == ERR_UNKNOWN_USER
        rc, table, _ = impl.alloc([3], [9], 5)                    # device free queue 4 5 2 3 0 1
        assert rc == OK and list(table[0]) == [4, 5, 2, 3, 0]
        # one host page free, user 3 needs 5: the host users go, oldest first, unless pinned
        assert impl.offload([3], [2])[0] == ERR_NO_SPACE
        rc, dropped = impl.offload([3])
        assert rc == OK and [int(d) for d in dropped] == [1, 2]
        rc, where, lens = impl.residency([1, 2, 3])
        assert list(where) == [0, 0, 2] and list(lens) == [0, 0, 9]
        assert impl.onboard([3]) == OK                            # device free queue 1 4 5 2 3 0
        rc, table, lens = impl.alloc([3], [0], 5)
        assert rc == OK and list(table[0]) == [1, 4, 5, 2, 3] and list(lens) == [9]
        assert impl.onboard([3]) == ERR_UNKNOWN_USER
        assert impl.offload([3, 3])[0] == ERR_INVALID
        assert impl.alloc([4], [2], 4)[0] == OK                   # takes the last device page
        assert impl.offload([4])[0] == OK
        assert impl.alloc([5], [2], 4)[0] == OK                   # and again
        before = impl.dump()
        assert impl.onboard([4]) == ERR_NO_SPACE and impl.dump() == before
        assert impl.evict_lru(1, [])[0] == OK                     # evicts user 3 (older)
        assert impl.onboard([4]) == OK
        rc, where, lens = impl.residency([3, 4, 5])
        assert list(where) == [0, 1, 1] and list(lens) == [0, 2, 2]


def test_host_tier_dump_load_roundtrip():
    from generative_recommender_sequence_amd import hstu
    c = hstu.KVCache.host_only(10, 4)
    assert c.host_attach(6) == OK
    assert c.alloc([5, 9], [9, 2], 8)[0] == OK
    assert c.offload([5])[0] == OK
    snap = c.dump()
    assert c.onboard([5]) == OK
    assert c.dump() != snap
    c.load(snap)
    assert c.dump() == snap
    plain = hstu.KVCache.host_only(10, 4)
    with pytest.raises(hstu.HstuError):
        plain.load(snap)                       # version 2 needs a host tier
    m = KVModel(10, 4)
    m.host_attach(6)
    m.alloc([5, 9], [9, 2], 8)
    m.offload([5])
    assert m.dump() == snap


def test_library_dump_load_roundtrip():
    from generative_recommender_sequence_amd import hstu
    c = hstu.KVCache.host_only(12, 4, list(range(11, -1, -1)))
    assert c.alloc([5, 9], [9, 2], 8)[0] == OK
    snap = c.dump()
    assert c.alloc([7], [13], 8)[0] == OK
    assert c.evict_lru(8, [7])[0] == OK
    assert c.dump() != snap
    c.load(snap)
    assert c.dump() == snap
    bad = bytearray(snap)
    bad[-4:] = bad[-8:-4]                      # a page listed twice
    with pytest.raises(hstu.HstuError):
        c.load(bytes(bad))
    assert c.dump() == snap                    # unchanged after a failed load


def test_exhaustion_and_all_pinned():
    for impl in _impls(5, 4, [4, 3, 2, 1, 0], with_lib=True).values():
        rc, table, lens = impl.alloc([1, 2], [8, 8], 4)          # 2 + 2 pages
        assert rc == OK and [list(r[:2]) for r in table] == [[4, 3], [2, 1]]
        before = impl.dump()
        rc, *_ = impl.alloc([3], [8], 4)                         # needs 2, 1 free
        assert rc == ERR_NO_SPACE and impl.dump() == before
        rc, ev = impl.evict_lru(3, [1, 2])                        # all pinned
        assert rc == ERR_NO_SPACE and len(ev) == 0 and impl.dump() == before
        rc, ev = impl.evict_lru(3, [2])                           # evicts user 1 (older tick)
        assert rc == OK and list(ev) == [1]
        rc, table, lens = impl.alloc([3], [8], 4)
        assert rc == OK and list(table[0][:2]) == [0, 4]          # FIFO: 0 first, then 1's pages
        assert impl.truncate(99, 0) == ERR_UNKNOWN_USER
        assert impl.truncate(3, 9) == ERR_INVALID
        assert impl.truncate(3, 3) == OK
        rc, lens = impl.lookup([3, 2, 7])
        assert rc == OK and list(lens) == [3, 8, 0]
        rc, *_ = impl.alloc([5, 5], [1, 1], 4)
        assert rc == ERR_INVALID


def test_lru_order_and_tie_break():
    for impl in _impls(8, 1, None, with_lib=True).values():
        assert impl.alloc([30, 10, 20], [2, 2, 2], 8)[0] == OK
        assert impl.lookup([30])[0] == OK                         # 30 becomes most recent
        rc, ev = impl.evict_lru(6, [])
        assert rc == OK and list(ev) == [10, 20]

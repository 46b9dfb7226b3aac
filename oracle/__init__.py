"""CPU oracle for the HSTU block forward with a paged KV cache.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing here imports the HIP library
or its package, and the HIP library never calls into this directory.

Pieces:
  hstu_oracle.c   one layer / the attention, in double (plain definition)
  kv_oracle.c     cache metadata (allocator, LRU, canonical dump)
  brute.py        an independent float64 brute force (dense padded masks)
  this file       ctypes wrappers, a layer-stack runner, and the pool-byte
                  placement model of the KV table layout

Every function here is pinned to something other than itself; the pins and
what each one fixes are listed at the top of tests/oracle_pins.py, and
tests/test_oracle.py also proves that a planted mistake in any part of the
oracle (compile flag ORACLE_MUTANT) fails at least one pin.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["hstu_oracle.c", "kv_oracle.c"]

OK, ERR_INVALID, ERR_NO_SPACE, ERR_UNKNOWN_USER = 0, 1, 2, 3


def lib_path(mutant: int = 0) -> str:
    if mutant == 0 and os.environ.get("ORACLE_LIBRARY"):   # a prebuilt variant (the sanitizer test's)
        return os.environ["ORACLE_LIBRARY"]
    name = "liboracle.so" if mutant == 0 else f"liboracle_mutant{mutant}.so"
    return os.path.join(HERE, "_build", name)


def build(mutant: int = 0, force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    out = lib_path(mutant)
    srcs = [os.path.join(HERE, s) for s in SOURCES]
    if mutant == 0 and os.environ.get("ORACLE_LIBRARY"):
        return out
    if not force and os.path.exists(out) and \
            os.path.getmtime(out) >= max(os.path.getmtime(f) for f in srcs):
        return out
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=gnu11", "-fno-fast-math",
           f"-DORACLE_MUTANT={mutant}", "-o", tmp] + srcs + ["-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_LIBS: Dict[int, ctypes.CDLL] = {}


def load(mutant: int = 0) -> ctypes.CDLL:
    if mutant in _LIBS:
        return _LIBS[mutant]
    path = build(mutant, force=False)
    lib = ctypes.CDLL(path)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f64p = ctypes.POINTER(ctypes.c_double)
    f32p = ctypes.POINTER(ctypes.c_float)
    vp = ctypes.c_void_p
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_threads.argtypes = []
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_layer_norm.restype = None
    lib.oracle_layer_norm.argtypes = [f64p, ctypes.c_int, ctypes.c_double, f64p]
    lib.oracle_bucket.restype = ctypes.c_int
    lib.oracle_bucket.argtypes = [ctypes.c_int64, ctypes.c_int]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [ctypes.c_int] * 3 + [i64p] * 3 + [i64p, f64p] + [f64p] * 4 + [ctypes.c_int, f64p]
    lib.oracle_layer.restype = ctypes.c_int
    lib.oracle_layer.argtypes = ([ctypes.c_int] * 4 + [ctypes.c_double] + [i64p] * 3 + [f64p] +
                                 [f64p] + [f32p] * 3 + [ctypes.c_int, i64p, f64p, f64p] + [f64p] * 8)
    lib.oracle_layer_backward.restype = ctypes.c_int
    lib.oracle_layer_backward.argtypes = ([ctypes.c_int] * 4 + [ctypes.c_double, i64p, i64p, f64p] + [f64p] * 4 +
                                          [ctypes.c_int] + [f64p] * 5)
    lib.oracle_head.restype = ctypes.c_int
    lib.oracle_head.argtypes = [f64p, ctypes.c_int64, ctypes.c_int, i32p, ctypes.c_int64, ctypes.c_int,
                                ctypes.c_int] + [f64p] * 5
    lib.oracle_kv_create.restype = vp
    lib.oracle_kv_create.argtypes = [ctypes.c_int32, ctypes.c_int32, i32p]
    lib.oracle_kv_destroy.restype = None
    lib.oracle_kv_destroy.argtypes = [vp]
    lib.oracle_kv_lookup.restype = ctypes.c_int
    lib.oracle_kv_lookup.argtypes = [vp, i64p, ctypes.c_int32, i32p]
    lib.oracle_kv_evict_lru.restype = ctypes.c_int
    lib.oracle_kv_evict_lru.argtypes = [vp, ctypes.c_int32, i64p, ctypes.c_int32, i64p, ctypes.c_int32, i32p]
    lib.oracle_kv_lru_victims.restype = ctypes.c_int
    lib.oracle_kv_lru_victims.argtypes = [vp, ctypes.c_int32, i64p, ctypes.c_int32, i64p, ctypes.c_int32, i32p]
    lib.oracle_kv_alloc.restype = ctypes.c_int
    lib.oracle_kv_alloc.argtypes = [vp, i64p, i32p, ctypes.c_int32, i32p, ctypes.c_int32, i32p]
    lib.oracle_kv_truncate.restype = ctypes.c_int
    lib.oracle_kv_truncate.argtypes = [vp, ctypes.c_int64, ctypes.c_int32]
    lib.oracle_kv_dump.restype = ctypes.c_int64
    lib.oracle_kv_dump.argtypes = [vp, ctypes.c_void_p, ctypes.c_int64]
    lib.oracle_kv_host_attach.restype = ctypes.c_int
    lib.oracle_kv_host_attach.argtypes = [vp, ctypes.c_int32]
    lib.oracle_kv_residency.restype = ctypes.c_int
    lib.oracle_kv_residency.argtypes = [vp, i64p, ctypes.c_int32, i32p, i32p]
    lib.oracle_kv_offload.restype = ctypes.c_int
    lib.oracle_kv_offload.argtypes = [vp, i64p, ctypes.c_int32, i64p, ctypes.c_int32, i64p, ctypes.c_int32,
                                      i32p]
    lib.oracle_kv_onboard.restype = ctypes.c_int
    lib.oracle_kv_onboard.argtypes = [vp, i64p, ctypes.c_int32]
    _LIBS[mutant] = lib
    return lib


def _p(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def offsets(lengths: Sequence[int]) -> np.ndarray:
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return off


# ---------------------------------------------------------------------------
# elementwise pieces
# ---------------------------------------------------------------------------

def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return load(0).oracle_threads()


def set_threads(n: int):
    """Threads of the oracle's parallel loops from now on (e.g. 1)."""
    load(0).oracle_set_threads(int(n))


def silu(z: float, mutant: int = 0) -> float:
    return load(mutant).oracle_silu(float(z))


def layer_norm(x: np.ndarray, eps: float, mutant: int = 0) -> np.ndarray:
    x = _f64(x)
    out = np.empty_like(x)
    load(mutant).oracle_layer_norm(_p(x, ctypes.c_double), x.size, float(eps), _p(out, ctypes.c_double))
    return out


def bucket(delta: int, num_buckets: int, mutant: int = 0) -> int:
    return load(mutant).oracle_bucket(int(delta), int(num_buckets))


# ---------------------------------------------------------------------------
# attention and a layer
# ---------------------------------------------------------------------------

def attention(q, k, v, new_len, start, kv_len, n_targets, norm_n, rab, num_heads, head_dim,
              mutant: int = 0) -> np.ndarray:
    """q [N_new, H*dh]; k, v [sum L_u, H*dh] (all positions of each user, jagged);
    returns o [N_new, H*dh] = (1/n_u) sum SiLU(q.k + rab) v under the mask."""
    lib = load(mutant)
    B = len(new_len)
    q, k, v = _f64(q), _f64(k), _f64(v)
    rab = _f64(rab)
    q_off, kv_off = offsets(new_len), offsets(kv_len)
    start, n_targets, norm_n = _i64(start), _i64(n_targets), _f64(norm_n)
    o = np.zeros((int(q_off[-1]), num_heads * head_dim), dtype=np.float64)
    rc = lib.oracle_attention(B, num_heads, head_dim, _p(q_off, ctypes.c_int64), _p(start, ctypes.c_int64),
                              _p(kv_off, ctypes.c_int64), _p(n_targets, ctypes.c_int64),
                              _p(norm_n, ctypes.c_double), _p(q, ctypes.c_double), _p(k, ctypes.c_double),
                              _p(v, ctypes.c_double), _p(rab, ctypes.c_double), len(rab),
                              _p(o, ctypes.c_double))
    if rc != OK:
        raise ValueError(f"oracle_attention rc={rc}")
    return o


def layer(x, w1, w2, rab, new_len, start, n_targets, norm_n, hist_k, hist_v, num_heads, head_dim,
          eps=1e-5, mutant: int = 0) -> Dict[str, np.ndarray]:
    """One HSTU layer for the new tokens of a jagged batch.

    x [N_new, d]; hist_k/hist_v [sum c_u, H*dh] cached K/V of each user
    (c_u = start[u]).  Everything is taken as float64.  Returns float64 arrays
    xhat, u, v, q, k, o, g, y."""
    lib = load(mutant)
    B = len(new_len)
    x = _f64(x)
    n_new, d = x.shape
    inner = num_heads * head_dim
    q_off = offsets(new_len)
    assert q_off[-1] == n_new
    start, n_targets, norm_n = _i64(start), _i64(n_targets), _f64(norm_n)
    hist_off = offsets(start)
    hk = _f64(hist_k).reshape(-1)
    hv = _f64(hist_v).reshape(-1)
    if hk.size == 0:
        hk = np.zeros(1, np.float64)
        hv = np.zeros(1, np.float64)
    out = {name: np.zeros((n_new, d if name in ("xhat", "y") else inner), np.float64)
           for name in ("xhat", "u", "v", "q", "k", "o", "g", "y")}
    rc = lib.oracle_layer(B, d, num_heads, head_dim, float(eps), _p(q_off, ctypes.c_int64),
                          _p(start, ctypes.c_int64), _p(n_targets, ctypes.c_int64), _p(norm_n, ctypes.c_double),
                          _p(x, ctypes.c_double), _p(_f32(w1), ctypes.c_float), _p(_f32(w2), ctypes.c_float),
                          _p(_f32(rab), ctypes.c_float), len(rab), _p(hist_off, ctypes.c_int64),
                          _p(hk, ctypes.c_double), _p(hv, ctypes.c_double),
                          *[_p(out[n], ctypes.c_double) for n in ("xhat", "u", "v", "q", "k", "o", "g", "y")])
    if rc != OK:
        raise ValueError(f"oracle_layer rc={rc}")
    return out


def layer_backward(x, w1, w2, rab, lengths, n_targets, norm_n, dy, num_heads, head_dim, eps=1e-5,
                   mutant: int = 0) -> Dict[str, np.ndarray]:
    """Gradients of one layer (every position computed, no cache) for
    dL/dY = dy: {"x", "w1", "w2", "rab"} in float64 (see
    oracle_layer_backward in hstu_oracle.c)."""
    x, w1, w2, rab, dy = (_f64(t) for t in (x, w1, w2, rab, dy))
    q_off = offsets(lengths)
    nt = _i64(n_targets)
    nn = _f64(norm_n)
    d = x.shape[1]
    out = {"x": np.zeros_like(x), "w1": np.zeros_like(w1), "w2": np.zeros_like(w2), "rab": np.zeros_like(rab)}
    rc = load(mutant).oracle_layer_backward(
        len(lengths), d, num_heads, head_dim, float(eps), _p(q_off, ctypes.c_int64), _p(nt, ctypes.c_int64),
        _p(nn, ctypes.c_double), _p(x, ctypes.c_double), _p(w1, ctypes.c_double), _p(w2, ctypes.c_double),
        _p(rab, ctypes.c_double), len(rab), _p(dy, ctypes.c_double), _p(out["x"], ctypes.c_double),
        _p(out["w1"], ctypes.c_double), _p(out["w2"], ctypes.c_double), _p(out["rab"], ctypes.c_double))
    if rc != OK:
        raise ValueError(f"oracle_layer_backward: status {rc}")
    return out


def head(y, rows, a, b, w, c, mutant: int = 0) -> np.ndarray:
    """Multitask ranking head: logits [len(rows)][tasks] of rows `rows` of y
    [*][d]; a [tasks][d][hidden], b [tasks][hidden], w [tasks][hidden], c
    [tasks] (see oracle_head in hstu_oracle.c for the formula)."""
    y, a, b, w, c = (_f64(t) for t in (y, a, b, w, c))
    rows = np.ascontiguousarray(np.asarray(rows, np.int32))
    tasks, d, hidden = a.shape
    out = np.zeros((len(rows), tasks))
    rc = load(mutant).oracle_head(_p(y, ctypes.c_double), y.shape[0], d, _p(rows, ctypes.c_int32), len(rows),
                                  tasks, hidden, _p(a, ctypes.c_double), _p(b, ctypes.c_double),
                                  _p(w, ctypes.c_double), _p(c, ctypes.c_double), _p(out, ctypes.c_double))
    if rc != OK:
        raise ValueError(f"oracle_head: status {rc}")
    return out


def candidate_rows(new_len, n_targets) -> np.ndarray:
    """Rows of the new-token matrix holding each user's candidates (the last
    min(T_u, t_u) new tokens of each user), in batch order."""
    off = offsets(new_len)
    return np.concatenate([np.arange(off[b + 1] - min(int(n_targets[b]), int(new_len[b])), off[b + 1])
                           for b in range(len(new_len))] + [np.zeros(0, np.int64)]).astype(np.int32)


class UserCache:
    """The oracle's own per-user, per-layer K/V store (contiguous, logical order)."""

    def __init__(self, num_layers: int, inner: int):
        self.num_layers = num_layers
        self.inner = inner
        self.k: Dict[int, List[np.ndarray]] = {}
        self.v: Dict[int, List[np.ndarray]] = {}

    def length(self, user) -> int:
        return 0 if user not in self.k else len(self.k[user][0])

    def get(self, user, layer_idx):
        if user not in self.k:
            e = np.zeros((0, self.inner), np.float64)
            return e, e
        return self.k[user][layer_idx], self.v[user][layer_idx]

    def append(self, user, layer_idx, k_new, v_new, store=np.float64):
        if user not in self.k:
            self.k[user] = [np.zeros((0, self.inner), np.float64) for _ in range(self.num_layers)]
            self.v[user] = [np.zeros((0, self.inner), np.float64) for _ in range(self.num_layers)]
        self.k[user][layer_idx] = np.concatenate([self.k[user][layer_idx], k_new.astype(store)])
        self.v[user][layer_idx] = np.concatenate([self.v[user][layer_idx], v_new.astype(store)])


def stack(layers, x_users: List[np.ndarray], n_targets, norm_n, num_heads, head_dim, eps=1e-5,
          cache: Optional[UserCache] = None, users=None, round_kv=None, mutant: int = 0,
          return_all: bool = False):
    """Run the layer stack on the new tokens of each user.

    x_users[u] is [t_u, d] (the new tokens); the cached length of user u is
    cache.length(users[u]) (0 without a cache).  New K/V are appended to the
    cache after each layer (optionally passed through round_kv, e.g. to
    emulate a storage precision).  Returns the final Y per user (and per
    layer outputs if return_all)."""
    B = len(x_users)
    new_len = [len(xu) for xu in x_users]
    starts = [cache.length(users[u]) if cache is not None else 0 for u in range(B)]
    x = np.concatenate(x_users, axis=0).astype(np.float64) if B else np.zeros((0, 1), np.float64)
    per_layer = []
    q_off = offsets(new_len)
    for li, lw in enumerate(layers):
        if cache is not None:
            hk = [cache.get(users[u], li)[0] for u in range(B)]
            hv = [cache.get(users[u], li)[1] for u in range(B)]
        else:
            hk = [np.zeros((0, num_heads * head_dim), np.float64)] * B
            hv = hk
        hk = np.concatenate(hk) if B else np.zeros((0, num_heads * head_dim), np.float64)
        hv = np.concatenate(hv) if B else hk
        out = layer(x, lw.w1, lw.w2, lw.rab, new_len, starts, n_targets, norm_n, hk, hv,
                    num_heads, head_dim, eps, mutant)
        if cache is not None:
            for u in range(B):
                kk = out["k"][q_off[u]:q_off[u + 1]]
                vv = out["v"][q_off[u]:q_off[u + 1]]
                if round_kv is not None:
                    kk, vv = round_kv(kk), round_kv(vv)
                cache.append(users[u], li, kk, vv)
        per_layer.append(out)
        x = out["y"]
    ys = [per_layer[-1]["y"][q_off[u]:q_off[u + 1]] for u in range(B)] if layers else x_users
    return (ys, per_layer) if return_all else ys


# ---------------------------------------------------------------------------
# KV table: allocator metadata and pool placement
# ---------------------------------------------------------------------------

class KVOracle:
    """ctypes wrapper of the oracle allocator (kv_oracle.c)."""

    def __init__(self, num_pages: int, page_size: int, free_order=None, mutant: int = 0):
        self.lib = load(mutant)
        fo = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        self._fo = fo
        self.h = self.lib.oracle_kv_create(num_pages, page_size,
                                           None if fo is None else _p(fo, ctypes.c_int32))
        if not self.h:
            raise ValueError("oracle_kv_create failed")
        self.page_size = page_size

    def __del__(self):
        if getattr(self, "h", None):
            self.lib.oracle_kv_destroy(self.h)
            self.h = None

    def lookup(self, users):
        u = _i64(users)
        out = np.zeros(len(u), np.int32)
        rc = self.lib.oracle_kv_lookup(self.h, _p(u, ctypes.c_int64), len(u), _p(out, ctypes.c_int32))
        return rc, out

    def evict_lru(self, pages_needed, pinned, cap=1 << 16):
        p = _i64(pinned) if len(pinned) else np.zeros(1, np.int64)
        ev = np.zeros(max(cap, 1), np.int64)
        n = ctypes.c_int32(0)
        rc = self.lib.oracle_kv_evict_lru(self.h, int(pages_needed), _p(p, ctypes.c_int64), len(pinned),
                                          _p(ev, ctypes.c_int64), cap, ctypes.byref(n))
        return rc, ev[:n.value].copy()

    def lru_victims(self, pages_needed, pinned, cap=1 << 16):
        p = _i64(pinned) if len(pinned) else np.zeros(1, np.int64)
        ev = np.zeros(max(cap, 1), np.int64)
        n = ctypes.c_int32(0)
        rc = self.lib.oracle_kv_lru_victims(self.h, int(pages_needed), _p(p, ctypes.c_int64), len(pinned),
                                            _p(ev, ctypes.c_int64), cap, ctypes.byref(n))
        return rc, ev[:n.value].copy()

    def alloc(self, users, n_new, max_pages):
        u = _i64(users)
        nn = np.ascontiguousarray(n_new, dtype=np.int32)
        pt = np.full((max(len(u), 1), max(max_pages, 1)), -7, np.int32)
        kl = np.zeros(max(len(u), 1), np.int32)
        rc = self.lib.oracle_kv_alloc(self.h, _p(u, ctypes.c_int64), _p(nn, ctypes.c_int32), len(u),
                                      _p(pt, ctypes.c_int32), max_pages, _p(kl, ctypes.c_int32))
        return rc, pt[:len(u), :max_pages].copy(), kl[:len(u)].copy()

    def truncate(self, user, new_len):
        return self.lib.oracle_kv_truncate(self.h, int(user), int(new_len))

    def dump(self) -> bytes:
        n = self.lib.oracle_kv_dump(self.h, None, 0)
        buf = (ctypes.c_uint8 * n)()
        n2 = self.lib.oracle_kv_dump(self.h, buf, n)
        assert n2 == n
        return bytes(buf)

    # host tier
    def host_attach(self, host_pages):
        return self.lib.oracle_kv_host_attach(self.h, int(host_pages))

    def residency(self, users):
        u = _i64(users) if len(users) else np.zeros(1, np.int64)
        where = np.zeros(max(len(users), 1), np.int32)
        ln = np.zeros(max(len(users), 1), np.int32)
        rc = self.lib.oracle_kv_residency(self.h, _p(u, ctypes.c_int64), len(users), _p(where, ctypes.c_int32),
                                          _p(ln, ctypes.c_int32))
        return rc, where[:len(users)].copy(), ln[:len(users)].copy()

    def offload(self, users, pinned=(), cap=1 << 16):
        u = _i64(users) if len(users) else np.zeros(1, np.int64)
        p = _i64(pinned) if len(pinned) else np.zeros(1, np.int64)
        dr = np.zeros(max(cap, 1), np.int64)
        n = ctypes.c_int32(0)
        rc = self.lib.oracle_kv_offload(self.h, _p(u, ctypes.c_int64), len(users), _p(p, ctypes.c_int64),
                                        len(pinned), _p(dr, ctypes.c_int64), cap, ctypes.byref(n))
        return rc, dr[:n.value].copy()

    def onboard(self, users):
        u = _i64(users) if len(users) else np.zeros(1, np.int64)
        return self.lib.oracle_kv_onboard(self.h, _p(u, ctypes.c_int64), len(users))


def pool_offset(layer_idx, page, head, slot, num_pages, num_heads, page_size, head_dim):
    """Element offset of (layer, page, head, slot, 0) in a K or V pool laid out
    [layers][pages][heads][page_size][head_dim]."""
    return ((((layer_idx * num_pages + page) * num_heads + head) * page_size + slot) * head_dim)


def pool_place(pool: np.ndarray, layer_idx: int, page_table_row, start_pos: int, rows: np.ndarray,
               num_pages: int, num_heads: int, page_size: int, head_dim: int) -> None:
    """Write rows [n, H*dh] of one user at positions start_pos.. into the flat pool."""
    for t in range(rows.shape[0]):
        pos = start_pos + t
        page = int(page_table_row[pos // page_size])
        slot = pos % page_size
        for h in range(num_heads):
            off = pool_offset(layer_idx, page, h, slot, num_pages, num_heads, page_size, head_dim)
            pool[off:off + head_dim] = rows[t, h * head_dim:(h + 1) * head_dim]


def pool_read(pool: np.ndarray, layer_idx: int, page_table_row, length: int, num_pages: int,
              num_heads: int, page_size: int, head_dim: int) -> np.ndarray:
    """Read positions 0..length-1 of one user from the flat pool -> [length, H*dh]."""
    out = np.zeros((length, num_heads * head_dim), dtype=pool.dtype)
    for pos in range(length):
        page = int(page_table_row[pos // page_size])
        slot = pos % page_size
        for h in range(num_heads):
            off = pool_offset(layer_idx, page, h, slot, num_pages, num_heads, page_size, head_dim)
            out[pos, h * head_dim:(h + 1) * head_dim] = pool[off:off + head_dim]
    return out

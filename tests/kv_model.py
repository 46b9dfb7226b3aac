"""Pure-Python model of the paged KV-cache metadata (the third, independent
implementation of the allocator rules; see oracle/kv_oracle.c for the rules
and the canonical dump format)."""
from __future__ import annotations

import struct
from collections import deque

OK, ERR_INVALID, ERR_NO_SPACE, ERR_UNKNOWN_USER = 0, 1, 2, 3


def _ceil(a, b):
    return -(-a // b)


class KVModel:
    def __init__(self, num_pages, page_size, free_order=None):
        self.num_pages = num_pages
        self.page_size = page_size
        self.free = deque(range(num_pages) if free_order is None else [int(p) for p in free_order])
        self.users = {}  # id -> [len, tick, pages]
        self.tick = 0

    def lookup(self, ids):
        ids = [int(i) for i in ids]
        if len(set(ids)) != len(ids):
            return ERR_INVALID, None
        out = []
        for i in ids:
            if i in self.users:
                self.tick += 1
                self.users[i][1] = self.tick
                out.append(self.users[i][0])
            else:
                out.append(0)
        return OK, out

    def evict_lru(self, pages_needed, pinned, cap=1 << 16):
        if pages_needed < 0:
            return ERR_INVALID, []
        if len(self.free) >= pages_needed:
            return OK, []
        pinned = set(int(p) for p in pinned)
        cands = sorted((u for u in self.users if u not in pinned),
                       key=lambda u: (self.users[u][1], u))
        have, chosen = len(self.free), []
        for u in cands:
            if have >= pages_needed:
                break
            chosen.append(u)
            have += len(self.users[u][2])
        if have < pages_needed:
            return ERR_NO_SPACE, []
        if len(chosen) > cap:
            return ERR_INVALID, []
        for u in chosen:
            self.free.extend(self.users.pop(u)[2])
        return OK, chosen

    def alloc(self, ids, n_new, max_pages):
        ids = [int(i) for i in ids]
        if len(set(ids)) != len(ids) or max_pages < 0:
            return ERR_INVALID, None, None
        need = 0
        for i, n in zip(ids, n_new):
            if n < 0:
                return ERR_INVALID, None, None
            ln = self.users[i][0] if i in self.users else 0
            if _ceil(ln + n, self.page_size) > max_pages:
                return ERR_INVALID, None, None
            need += _ceil(ln + n, self.page_size) - _ceil(ln, self.page_size)
        if need > len(self.free):
            return ERR_NO_SPACE, None, None
        table, lens = [], []
        for i, n in zip(ids, n_new):
            if i not in self.users:
                self.users[i] = [0, 0, []]
            rec = self.users[i]
            while len(rec[2]) < _ceil(rec[0] + n, self.page_size):
                rec[2].append(self.free.popleft())
            rec[0] += n
            self.tick += 1
            rec[1] = self.tick
            table.append(rec[2] + [-1] * (max_pages - len(rec[2])))
            lens.append(rec[0])
        return OK, table, lens

    def truncate(self, user, new_len):
        user = int(user)
        if user not in self.users:
            return ERR_UNKNOWN_USER
        rec = self.users[user]
        if new_len < 0 or new_len > rec[0]:
            return ERR_INVALID
        keep = _ceil(new_len, self.page_size)
        self.free.extend(rec[2][keep:])
        rec[2] = rec[2][:keep]
        rec[0] = new_len
        return OK

    def dump(self) -> bytes:
        out = struct.pack("<IIiiqii", 0x564B5348, 1, self.num_pages, self.page_size, self.tick,
                          len(self.users), len(self.free))
        for u in sorted(self.users):
            ln, tk, pages = self.users[u]
            out += struct.pack("<qiqi", u, ln, tk, len(pages))
            out += struct.pack(f"<{len(pages)}i", *pages)
        out += struct.pack(f"<{len(self.free)}i", *self.free)
        return out

    def check_invariants(self):
        owned = [p for rec in self.users.values() for p in rec[2]]
        allp = owned + list(self.free)
        assert sorted(allp) == list(range(self.num_pages)), "every page exactly once"
        for rec in self.users.values():
            assert len(rec[2]) == _ceil(rec[0], self.page_size)


def random_ops(rng, n_ops, num_users=12, max_new=70):
    """A seeded sequence of cache operations (used against all implementations)."""
    ops = []
    for _ in range(n_ops):
        kind = rng.choice(["lookup", "alloc", "alloc", "evict", "truncate"])
        if kind == "lookup":
            ids = rng.choice(num_users, size=rng.integers(0, 5), replace=False) + 1
            ops.append(("lookup", [int(i) for i in ids]))
        elif kind == "alloc":
            B = int(rng.integers(0, 5))
            ids = rng.choice(num_users, size=B, replace=False) + 1
            nn = rng.integers(0, max_new, size=B)
            ops.append(("alloc", [int(i) for i in ids], [int(n) for n in nn], int(rng.integers(3, 12))))
        elif kind == "evict":
            pinned = rng.choice(num_users, size=rng.integers(0, 4), replace=False) + 1
            ops.append(("evict", int(rng.integers(0, 40)), [int(p) for p in pinned]))
        else:
            ops.append(("truncate", int(rng.integers(1, num_users + 1)), int(rng.integers(0, 200))))
    return ops

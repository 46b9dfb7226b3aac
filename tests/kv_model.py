"""Pure-Python model of the paged KV-cache metadata, host tier included (the
third, independent implementation of the allocator rules; see
oracle/kv_oracle.c for the rules and the canonical dump format)."""
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
        self.host_pages = None  # host tier: pages, free queue, users
        self.host_free = deque()
        self.hosts = {}

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

    def evict_lru(self, pages_needed, pinned, cap=1 << 16, drop=True):
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
        for u in chosen if drop else ():
            self.free.extend(self.users.pop(u)[2])
        return OK, chosen

    def lru_victims(self, pages_needed, pinned, cap=1 << 16):
        return self.evict_lru(pages_needed, pinned, cap, drop=False)

    def alloc(self, ids, n_new, max_pages):
        ids = [int(i) for i in ids]
        if len(set(ids)) != len(ids) or max_pages < 0:
            return ERR_INVALID, None, None
        need = 0
        for i, n in zip(ids, n_new):
            if n < 0 or i in self.hosts:
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

    # host tier
    def host_attach(self, host_pages):
        if self.host_pages is not None or host_pages < 0:
            return ERR_INVALID
        self.host_pages = host_pages
        self.host_free = deque(range(host_pages))
        return OK

    def residency(self, ids):
        where, lens = [], []
        for i in (int(x) for x in ids):
            if i in self.users:
                where.append(1)
                lens.append(self.users[i][0])
            elif i in self.hosts:
                where.append(2)
                lens.append(self.hosts[i][0])
            else:
                where.append(0)
                lens.append(0)
        return OK, where, lens

    def offload(self, ids, pinned=(), cap=1 << 16):
        ids = [int(i) for i in ids]
        pinned = set(int(p) for p in pinned)
        if self.host_pages is None or len(set(ids)) != len(ids):
            return ERR_INVALID, []
        if any(i not in self.users for i in ids):
            return ERR_UNKNOWN_USER, []
        need = sum(len(self.users[i][2]) for i in ids)
        have, dropped = len(self.host_free), []
        for h in sorted((h for h in self.hosts if h not in pinned), key=lambda h: (self.hosts[h][1], h)):
            if have >= need:
                break
            dropped.append(h)
            have += len(self.hosts[h][2])
        if have < need:
            return ERR_NO_SPACE, []
        if len(dropped) > cap:
            return ERR_INVALID, []
        for h in dropped:
            self.host_free.extend(self.hosts.pop(h)[2])
        for i in ids:
            ln, tk, pages = self.users.pop(i)
            self.hosts[i] = [ln, tk, [self.host_free.popleft() for _ in pages]]
            self.free.extend(pages)
        return OK, dropped

    def onboard(self, ids):
        ids = [int(i) for i in ids]
        if self.host_pages is None or len(set(ids)) != len(ids):
            return ERR_INVALID
        if any(i not in self.hosts for i in ids):
            return ERR_UNKNOWN_USER
        if sum(len(self.hosts[i][2]) for i in ids) > len(self.free):
            return ERR_NO_SPACE
        for i in ids:
            ln, _, hpages = self.hosts.pop(i)
            self.tick += 1
            self.users[i] = [ln, self.tick, [self.free.popleft() for _ in hpages]]
            self.host_free.extend(hpages)
        return OK

    @staticmethod
    def _tier_bytes(users, free):
        out = b""
        for u in sorted(users):
            ln, tk, pages = users[u]
            out += struct.pack("<qiqi", u, ln, tk, len(pages))
            out += struct.pack(f"<{len(pages)}i", *pages)
        return out + struct.pack(f"<{len(free)}i", *free)

    def dump(self) -> bytes:
        version = 1 if self.host_pages is None else 2
        out = struct.pack("<IIiiqii", 0x564B5348, version, self.num_pages, self.page_size, self.tick,
                          len(self.users), len(self.free))
        out += self._tier_bytes(self.users, self.free)
        if self.host_pages is not None:
            out += struct.pack("<iii", self.host_pages, len(self.hosts), len(self.host_free))
            out += self._tier_bytes(self.hosts, self.host_free)
        return out

    def check_invariants(self):
        owned = [p for rec in self.users.values() for p in rec[2]]
        allp = owned + list(self.free)
        assert sorted(allp) == list(range(self.num_pages)), "every page exactly once"
        for rec in self.users.values():
            assert len(rec[2]) == _ceil(rec[0], self.page_size)
        if self.host_pages is not None:
            hp = [p for rec in self.hosts.values() for p in rec[2]] + list(self.host_free)
            assert sorted(hp) == list(range(self.host_pages)), "every host page exactly once"
            assert not set(self.users) & set(self.hosts), "a user on one tier only"


def random_ops(rng, n_ops, num_users=12, max_new=70, host_tier=False):
    """A seeded sequence of cache operations (used against all implementations)."""
    ops = []
    kinds = ["lookup", "alloc", "alloc", "evict", "truncate"]
    if host_tier:
        kinds += ["offload", "onboard", "residency", "victims"]
    for _ in range(n_ops):
        kind = rng.choice(kinds)
        if kind in ("offload", "onboard", "residency"):
            ids = rng.choice(num_users, size=rng.integers(0, 4), replace=False) + 1
            op = (kind, [int(i) for i in ids])
            if kind == "offload":
                op += ([int(p) for p in rng.choice(num_users, size=rng.integers(0, 4), replace=False) + 1],)
            ops.append(op)
            continue
        if kind == "lookup":
            ids = rng.choice(num_users, size=rng.integers(0, 5), replace=False) + 1
            ops.append(("lookup", [int(i) for i in ids]))
        elif kind == "alloc":
            B = int(rng.integers(0, 5))
            ids = rng.choice(num_users, size=B, replace=False) + 1
            nn = rng.integers(0, max_new, size=B)
            ops.append(("alloc", [int(i) for i in ids], [int(n) for n in nn], int(rng.integers(3, 12))))
        elif kind in ("evict", "victims"):
            pinned = rng.choice(num_users, size=rng.integers(0, 4), replace=False) + 1
            ops.append((kind, int(rng.integers(0, 40)), [int(p) for p in pinned]))
        else:
            ops.append(("truncate", int(rng.integers(1, num_users + 1)), int(rng.integers(0, 200))))
    return ops


def parse_dump(data: bytes) -> dict:
    """The canonical dump as {"tick", "users": {id: (len, tick, pages)}, "free",
    and with a host tier "host_pages", "host_users", "host_free"}."""
    magic, version, num_pages, page_size, tick, n_users, n_free = struct.unpack_from("<IIiiqii", data, 0)
    off = struct.calcsize("<IIiiqii")

    def tier(off, n_users, n_free):
        users = {}
        for _ in range(n_users):
            u, ln, tk, n = struct.unpack_from("<qiqi", data, off)
            off += struct.calcsize("<qiqi")
            users[u] = (ln, tk, list(struct.unpack_from(f"<{n}i", data, off)))
            off += 4 * n
        free = list(struct.unpack_from(f"<{n_free}i", data, off))
        return users, free, off + 4 * n_free

    out = {"version": version, "num_pages": num_pages, "page_size": page_size, "tick": tick}
    out["users"], out["free"], off = tier(off, n_users, n_free)
    if version == 2:
        out["host_pages"], nh, nhf = struct.unpack_from("<iii", data, off)
        out["host_users"], out["host_free"], off = tier(off + 12, nh, nhf)
    assert off == len(data)
    return out

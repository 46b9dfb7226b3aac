// Host metadata of the paged KV table: lookup, allocation, LRU eviction,
// truncation, the host tier (offload and onboard), canonical state dump/load.
//
// Follows "Deploying an HSTU Generative Recommender with NVIDIA Dynamo-Triton"
// (KV cache section: a paged KV data table in GPU memory with lookup,
// allocation, onboarding, append, offloading and eviction; the table spans GPU
// and host storage; older users evicted LRU-style when space is tight).
// Policy details the pages leave open, fixed here and in hstu.h: FIFO
// free-page queues (one per tier); users served in batch order; whole-user
// eviction in (tick, id) order skipping pinned users; all-or-nothing
// allocation, eviction, offload and onboard.
#include <algorithm>
#include <cstring>

#include "internal.h"

using hstu::fail;
using hstu::ok;

namespace {

int32_t pages_for(int64_t len, int32_t p) { return static_cast<int32_t>((len + p - 1) / p); }

bool distinct(const int64_t* ids, int32_t n) {
  std::vector<int64_t> v(ids, ids + n);
  std::sort(v.begin(), v.end());
  return std::adjacent_find(v.begin(), v.end()) == v.end();
}

template <typename T>
void put(std::vector<unsigned char>& out, T v) {
  unsigned char b[sizeof(T)];
  std::memcpy(b, &v, sizeof(T));
  out.insert(out.end(), b, b + sizeof(T));
}

template <typename T>
bool get(const unsigned char*& p, const unsigned char* end, T* v) {
  if (static_cast<size_t>(end - p) < sizeof(T)) return false;
  std::memcpy(v, p, sizeof(T));
  p += sizeof(T);
  return true;
}

constexpr uint32_t kMagic = 0x564B5348u;

std::vector<unsigned char> serialize(const hstu_kv_cache* c) {
  std::vector<unsigned char> out;
  put<uint32_t>(out, kMagic);
  put<uint32_t>(out, c->host_pages >= 0 ? 2u : 1u);
  put<int32_t>(out, c->num_pages);
  put<int32_t>(out, c->page_size);
  put<int64_t>(out, c->tick);
  put<int32_t>(out, static_cast<int32_t>(c->users.size()));
  put<int32_t>(out, static_cast<int32_t>(c->free_q.size()));
  std::vector<int64_t> ids;
  ids.reserve(c->users.size());
  for (const auto& kv : c->users) ids.push_back(kv.first);
  std::sort(ids.begin(), ids.end());
  for (int64_t id : ids) {
    const auto& u = c->users.at(id);
    put<int64_t>(out, id);
    put<int32_t>(out, u.len);
    put<int64_t>(out, u.tick);
    put<int32_t>(out, static_cast<int32_t>(u.pages.size()));
    for (int32_t p : u.pages) put<int32_t>(out, p);
  }
  for (int32_t p : c->free_q) put<int32_t>(out, p);
  if (c->host_pages >= 0) {
    put<int32_t>(out, c->host_pages);
    put<int32_t>(out, static_cast<int32_t>(c->host_users.size()));
    put<int32_t>(out, static_cast<int32_t>(c->host_free_q.size()));
    std::vector<int64_t> hids;
    for (const auto& kv : c->host_users) hids.push_back(kv.first);
    std::sort(hids.begin(), hids.end());
    for (int64_t id : hids) {
      const auto& u = c->host_users.at(id);
      put<int64_t>(out, id);
      put<int32_t>(out, u.len);
      put<int64_t>(out, u.tick);
      put<int32_t>(out, static_cast<int32_t>(u.pages.size()));
      for (int32_t p : u.pages) put<int32_t>(out, p);
    }
    for (int32_t p : c->host_free_q) put<int32_t>(out, p);
  }
  return out;
}

// Reads one tier's users and free queue; pages must cover 0..n_pages-1 once.
bool read_tier(const unsigned char*& p, const unsigned char* end, int32_t n_users, int32_t n_free,
               int32_t n_pages, int32_t page_size, int64_t tick,
               std::unordered_map<int64_t, hstu_kv_cache::User>* users, std::deque<int32_t>* fq) {
  std::vector<char> seen(static_cast<size_t>(n_pages), 0);
  int64_t last_id = 0;
  for (int32_t i = 0; i < n_users; ++i) {
    int64_t id = 0, utick = 0;
    int32_t ulen = 0, np = 0;
    if (!get(p, end, &id) || !get(p, end, &ulen) || !get(p, end, &utick) || !get(p, end, &np)) return false;
    if ((i > 0 && id <= last_id) || ulen < 0 || utick < 0 || utick > tick || np != pages_for(ulen, page_size))
      return false;
    last_id = id;
    hstu_kv_cache::User u;
    u.len = ulen;
    u.tick = utick;
    for (int32_t k = 0; k < np; ++k) {
      int32_t pg = 0;
      if (!get(p, end, &pg) || pg < 0 || pg >= n_pages || seen[pg]) return false;
      seen[pg] = 1;
      u.pages.push_back(pg);
    }
    users->emplace(id, std::move(u));
  }
  for (int32_t k = 0; k < n_free; ++k) {
    int32_t pg = 0;
    if (!get(p, end, &pg) || pg < 0 || pg >= n_pages || seen[pg]) return false;
    seen[pg] = 1;
    fq->push_back(pg);
  }
  for (char x : seen)
    if (!x) return false;
  return true;
}

}  // namespace

extern "C" {

hstu_status kv_cache_create(const hstu_kv_cache_desc* d, hstu_kv_cache** out) {
  if (!d || !out) return fail(HSTU_ERR_INVALID, "kv_cache_create: null argument");
  *out = nullptr;
  if (d->num_layers <= 0 || d->num_heads <= 0 || d->head_dim <= 0 || d->page_size <= 0 ||
      d->num_pages < 0)
    return fail(HSTU_ERR_INVALID, "kv_cache_create: non-positive geometry");
  if (d->dtype != HSTU_F32 && d->dtype != HSTU_BF16)
    return fail(HSTU_ERR_INVALID, "kv_cache_create: unknown dtype");
  if ((d->k_pool == nullptr) != (d->v_pool == nullptr))
    return fail(HSTU_ERR_INVALID, "kv_cache_create: give both pools or neither");
  if (d->head_dim % 8 != 0)
    return fail(HSTU_ERR_UNSUPPORTED, "kv_cache_create: head_dim must be a multiple of 8");
  if (d->initial_free_order) {
    std::vector<char> seen(static_cast<size_t>(d->num_pages), 0);
    for (int32_t i = 0; i < d->num_pages; ++i) {
      int32_t p = d->initial_free_order[i];
      if (p < 0 || p >= d->num_pages || seen[p])
        return fail(HSTU_ERR_INVALID, "kv_cache_create: initial_free_order is not a permutation");
      seen[p] = 1;
    }
  }
  auto* c = new hstu_kv_cache();
  c->num_layers = d->num_layers;
  c->num_heads = d->num_heads;
  c->head_dim = d->head_dim;
  c->page_size = d->page_size;
  c->num_pages = d->num_pages;
  c->dtype = d->dtype;
  c->k_pool = d->k_pool;
  c->v_pool = d->v_pool;
  for (int32_t i = 0; i < d->num_pages; ++i)
    c->free_q.push_back(d->initial_free_order ? d->initial_free_order[i] : i);
  *out = c;
  return ok();
}

hstu_status kv_cache_destroy(hstu_kv_cache* c) {
  delete c;
  return ok();
}

hstu_status kv_lookup(hstu_kv_cache* c, const int64_t* users, int32_t B, int32_t* cached_len) {
  if (!c || B < 0 || (B > 0 && (!users || !cached_len)))
    return fail(HSTU_ERR_INVALID, "kv_lookup: bad arguments");
  if (!distinct(users, B)) return fail(HSTU_ERR_INVALID, "kv_lookup: duplicate users");
  for (int32_t b = 0; b < B; ++b) {
    auto it = c->users.find(users[b]);
    if (it == c->users.end()) {
      cached_len[b] = 0;
    } else {
      cached_len[b] = it->second.len;
      it->second.tick = ++c->tick;
    }
  }
  return ok();
}

namespace {
// The unpinned device-resident users, ascending (tick, id), that must go for
// the free queue to reach pages_needed (none if it already does).
hstu_status lru_selection(const hstu_kv_cache* c, int32_t pages_needed, const int64_t* pinned,
                          int32_t n_pinned, int32_t cap, std::vector<int64_t>& out, const char* who) {
  out.clear();
  int64_t have = static_cast<int64_t>(c->free_q.size());
  if (have >= pages_needed) return ok();
  std::vector<int64_t> pin(pinned, pinned + n_pinned);
  std::sort(pin.begin(), pin.end());
  std::vector<std::pair<int64_t, int64_t>> order;  // (tick, id)
  for (const auto& kv : c->users)
    if (!std::binary_search(pin.begin(), pin.end(), kv.first))
      order.emplace_back(kv.second.tick, kv.first);
  std::sort(order.begin(), order.end());
  size_t n = 0;
  while (have < pages_needed && n < order.size()) {
    have += static_cast<int64_t>(c->users.at(order[n].second).pages.size());
    out.push_back(order[n].second);
    ++n;
  }
  if (have < pages_needed)
    return fail(HSTU_ERR_NO_SPACE, std::string(who) + ": evicting every unpinned user is not enough");
  if (static_cast<int64_t>(n) > cap) return fail(HSTU_ERR_INVALID, std::string(who) + ": cap too small");
  return ok();
}
}  // namespace

hstu_status kv_evict_lru(hstu_kv_cache* c, int32_t pages_needed, const int64_t* pinned,
                         int32_t n_pinned, int64_t* evicted, int32_t cap, int32_t* n_evicted) {
  if (!c || pages_needed < 0 || n_pinned < 0 || cap < 0 || !n_evicted ||
      (n_pinned > 0 && !pinned) || (cap > 0 && !evicted))
    return fail(HSTU_ERR_INVALID, "kv_evict_lru: bad arguments");
  *n_evicted = 0;
  std::vector<int64_t> sel;
  hstu_status st = lru_selection(c, pages_needed, pinned, n_pinned, cap, sel, "kv_evict_lru");
  if (st != HSTU_OK) return st;
  for (size_t k = 0; k < sel.size(); ++k) {
    auto it = c->users.find(sel[k]);
    for (int32_t p : it->second.pages) c->free_q.push_back(p);
    evicted[k] = it->first;
    c->users.erase(it);
  }
  *n_evicted = static_cast<int32_t>(sel.size());
  return ok();
}

hstu_status kv_lru_victims(const hstu_kv_cache* c, int32_t pages_needed, const int64_t* pinned,
                           int32_t n_pinned, int64_t* victims, int32_t cap, int32_t* n_victims) {
  if (!c || pages_needed < 0 || n_pinned < 0 || cap < 0 || !n_victims ||
      (n_pinned > 0 && !pinned) || (cap > 0 && !victims))
    return fail(HSTU_ERR_INVALID, "kv_lru_victims: bad arguments");
  *n_victims = 0;
  std::vector<int64_t> sel;
  hstu_status st = lru_selection(c, pages_needed, pinned, n_pinned, cap, sel, "kv_lru_victims");
  if (st != HSTU_OK) return st;
  std::copy(sel.begin(), sel.end(), victims);
  *n_victims = static_cast<int32_t>(sel.size());
  return ok();
}

hstu_status kv_page_alloc(hstu_kv_cache* c, const int64_t* users, const int32_t* n_new, int32_t B,
                          int32_t* page_table, int32_t max_pages, int32_t* kv_len) {
  if (!c || B < 0 || max_pages < 0 ||
      (B > 0 && (!users || !n_new || !kv_len || (max_pages > 0 && !page_table))))
    return fail(HSTU_ERR_INVALID, "kv_page_alloc: bad arguments");
  if (!distinct(users, B)) return fail(HSTU_ERR_INVALID, "kv_page_alloc: duplicate users");
  int64_t need = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (n_new[b] < 0) return fail(HSTU_ERR_INVALID, "kv_page_alloc: negative n_new");
    if (c->host_users.count(users[b]))
      return fail(HSTU_ERR_INVALID, "kv_page_alloc: a user is on the host tier (onboard it first)");
    auto it = c->users.find(users[b]);
    int64_t len = it == c->users.end() ? 0 : it->second.len;
    int64_t after = len + n_new[b];
    if (after > INT32_MAX) return fail(HSTU_ERR_INVALID, "kv_page_alloc: length overflow");
    if (pages_for(after, c->page_size) > max_pages)
      return fail(HSTU_ERR_INVALID, "kv_page_alloc: a user needs more than max_pages pages");
    need += pages_for(after, c->page_size) - pages_for(len, c->page_size);
  }
  if (need > static_cast<int64_t>(c->free_q.size()))
    return fail(HSTU_ERR_NO_SPACE, "kv_page_alloc: not enough free pages");
  for (int32_t b = 0; b < B; ++b) {
    auto& u = c->users[users[b]];
    int32_t want = pages_for(static_cast<int64_t>(u.len) + n_new[b], c->page_size);
    while (static_cast<int32_t>(u.pages.size()) < want) {
      u.pages.push_back(c->free_q.front());
      c->free_q.pop_front();
    }
    u.len += n_new[b];
    u.tick = ++c->tick;
    kv_len[b] = u.len;
    for (int32_t k = 0; k < max_pages; ++k)
      page_table[static_cast<int64_t>(b) * max_pages + k] =
          k < static_cast<int32_t>(u.pages.size()) ? u.pages[k] : -1;
  }
  return ok();
}

hstu_status kv_truncate(hstu_kv_cache* c, int64_t user, int32_t new_len) {
  if (!c) return fail(HSTU_ERR_INVALID, "kv_truncate: null cache");
  auto it = c->users.find(user);
  if (it == c->users.end()) return fail(HSTU_ERR_UNKNOWN_USER, "kv_truncate: unknown user");
  auto& u = it->second;
  if (new_len < 0 || new_len > u.len) return fail(HSTU_ERR_INVALID, "kv_truncate: bad length");
  size_t keep = static_cast<size_t>(pages_for(new_len, c->page_size));
  for (size_t k = keep; k < u.pages.size(); ++k) c->free_q.push_back(u.pages[k]);
  u.pages.resize(keep);
  u.len = new_len;
  return ok();
}

hstu_status kv_free_pages(const hstu_kv_cache* c, int32_t* n_free) {
  if (!c || !n_free) return fail(HSTU_ERR_INVALID, "kv_free_pages: null argument");
  *n_free = static_cast<int32_t>(c->free_q.size());
  return ok();
}

hstu_status kv_page_table(const hstu_kv_cache* c, const int64_t* users, int32_t B,
                          int32_t* page_table, int32_t max_pages, int32_t* kv_len) {
  if (!c || B < 0 || max_pages < 0 ||
      (B > 0 && (!users || !kv_len || (max_pages > 0 && !page_table))))
    return fail(HSTU_ERR_INVALID, "kv_page_table: bad arguments");
  for (int32_t b = 0; b < B; ++b) {
    auto it = c->users.find(users[b]);
    if (it == c->users.end()) return fail(HSTU_ERR_UNKNOWN_USER, "kv_page_table: unknown user");
    if (static_cast<int32_t>(it->second.pages.size()) > max_pages)
      return fail(HSTU_ERR_INVALID, "kv_page_table: max_pages too small");
  }
  for (int32_t b = 0; b < B; ++b) {
    const auto& u = c->users.at(users[b]);
    kv_len[b] = u.len;
    for (int32_t k = 0; k < max_pages; ++k)
      page_table[static_cast<int64_t>(b) * max_pages + k] =
          k < static_cast<int32_t>(u.pages.size()) ? u.pages[k] : -1;
  }
  return ok();
}

hstu_status kv_state_dump(const hstu_kv_cache* c, void* buf, size_t cap, size_t* needed) {
  if (!c || !needed) return fail(HSTU_ERR_INVALID, "kv_state_dump: null argument");
  std::vector<unsigned char> bytes = serialize(c);
  *needed = bytes.size();
  if (buf && cap >= bytes.size()) std::memcpy(buf, bytes.data(), bytes.size());
  return ok();
}

hstu_status kv_state_load(hstu_kv_cache* c, const void* buf, size_t len) {
  if (!c || (!buf && len)) return fail(HSTU_ERR_INVALID, "kv_state_load: null argument");
  const unsigned char* p = static_cast<const unsigned char*>(buf);
  const unsigned char* end = p + len;
  uint32_t magic = 0, version = 0;
  int32_t num_pages = 0, page_size = 0, n_users = 0, n_free = 0;
  int64_t tick = 0;
  if (!get(p, end, &magic) || !get(p, end, &version) || !get(p, end, &num_pages) ||
      !get(p, end, &page_size) || !get(p, end, &tick) || !get(p, end, &n_users) ||
      !get(p, end, &n_free))
    return fail(HSTU_ERR_INVALID, "kv_state_load: truncated header");
  if (magic != kMagic || version != (c->host_pages >= 0 ? 2u : 1u))
    return fail(HSTU_ERR_INVALID, "kv_state_load: bad magic, or version does not match the host tier");
  if (num_pages != c->num_pages || page_size != c->page_size)
    return fail(HSTU_ERR_INVALID, "kv_state_load: geometry differs");
  if (n_users < 0 || n_free < 0 || tick < 0)
    return fail(HSTU_ERR_INVALID, "kv_state_load: negative counts");
  std::unordered_map<int64_t, hstu_kv_cache::User> users, host_users;
  std::deque<int32_t> fq, hfq;
  if (!read_tier(p, end, n_users, n_free, num_pages, page_size, tick, &users, &fq))
    return fail(HSTU_ERR_INVALID, "kv_state_load: inconsistent device tier");
  if (c->host_pages >= 0) {
    int32_t host_pages = 0, n_host_users = 0, n_host_free = 0;
    if (!get(p, end, &host_pages) || !get(p, end, &n_host_users) || !get(p, end, &n_host_free))
      return fail(HSTU_ERR_INVALID, "kv_state_load: truncated host header");
    if (host_pages != c->host_pages || n_host_users < 0 || n_host_free < 0)
      return fail(HSTU_ERR_INVALID, "kv_state_load: host geometry differs");
    if (!read_tier(p, end, n_host_users, n_host_free, host_pages, page_size, tick, &host_users, &hfq))
      return fail(HSTU_ERR_INVALID, "kv_state_load: inconsistent host tier");
    for (const auto& kv : host_users)
      if (users.count(kv.first)) return fail(HSTU_ERR_INVALID, "kv_state_load: a user on both tiers");
  }
  if (p != end) return fail(HSTU_ERR_INVALID, "kv_state_load: trailing bytes");
  c->tick = tick;
  c->users = std::move(users);
  c->free_q = std::move(fq);
  c->host_users = std::move(host_users);
  c->host_free_q = std::move(hfq);
  return ok();
}

// ---------------------------------------------------------------------------
// host tier
// ---------------------------------------------------------------------------

hstu_status kv_host_attach(hstu_kv_cache* c, void* host_k_pool, void* host_v_pool, int32_t host_pages) {
  if (!c || host_pages < 0) return fail(HSTU_ERR_INVALID, "kv_host_attach: bad arguments");
  if (c->host_pages >= 0) return fail(HSTU_ERR_INVALID, "kv_host_attach: a host tier is already attached");
  if ((host_k_pool == nullptr) != (host_v_pool == nullptr))
    return fail(HSTU_ERR_INVALID, "kv_host_attach: give both host pools or neither");
  if (c->k_pool && !host_k_pool)
    return fail(HSTU_ERR_INVALID, "kv_host_attach: a cache with device pools needs host pools");
  void* dk = nullptr;
  void* dv = nullptr;
  if (host_k_pool) {
    // the copy kernels address the host pools directly: they must be pinned
    if (hipHostGetDevicePointer(&dk, host_k_pool, 0) != hipSuccess ||
        hipHostGetDevicePointer(&dv, host_v_pool, 0) != hipSuccess) {
      (void)hipGetLastError();
      return fail(HSTU_ERR_INVALID, "kv_host_attach: host pools must be pinned host memory (hipHostMalloc)");
    }
  }
  c->host_pages = host_pages;
  c->host_k = dk;
  c->host_v = dv;
  c->host_free_q.clear();
  for (int32_t i = 0; i < host_pages; ++i) c->host_free_q.push_back(i);
  return ok();
}

hstu_status kv_residency(const hstu_kv_cache* c, const int64_t* users, int32_t B, int32_t* where, int32_t* len) {
  if (!c || B < 0 || (B > 0 && (!users || !where || !len)))
    return fail(HSTU_ERR_INVALID, "kv_residency: bad arguments");
  for (int32_t b = 0; b < B; ++b) {
    auto it = c->users.find(users[b]);
    if (it != c->users.end()) {
      where[b] = 1;
      len[b] = it->second.len;
      continue;
    }
    auto ht = c->host_users.find(users[b]);
    where[b] = ht != c->host_users.end() ? 2 : 0;
    len[b] = ht != c->host_users.end() ? ht->second.len : 0;
  }
  return ok();
}

namespace {
struct CopyCtx {
  int32_t n_pairs, layers;
  const void *sk, *sv;
  int64_t src_pages;
  void *dk, *dv;
  int64_t dst_pages, page_bytes;
  hipStream_t stream;
};
hipError_t launch_copy(const void* pairs, void* ctx) {
  auto* x = static_cast<CopyCtx*>(ctx);
  return hstu::launch_tier_copy(static_cast<const hstu::PagePair*>(pairs), x->n_pairs, x->layers, x->sk,
                                x->sv, x->src_pages, x->dk, x->dv, x->dst_pages, x->page_bytes, x->stream);
}
int64_t page_bytes(const hstu_kv_cache* c) {
  return static_cast<int64_t>(c->num_heads) * c->page_size * c->head_dim * (c->dtype == HSTU_BF16 ? 2 : 4);
}
}  // namespace

hstu_status kv_offload(hstu_kv_cache* c, const int64_t* users, int32_t n, const int64_t* pinned,
                       int32_t n_pinned, hipStream_t stream, int64_t* host_evicted, int32_t cap,
                       int32_t* n_host_evicted) {
  if (!c || n < 0 || n_pinned < 0 || cap < 0 || !n_host_evicted || (n > 0 && !users) ||
      (n_pinned > 0 && !pinned) || (cap > 0 && !host_evicted))
    return fail(HSTU_ERR_INVALID, "kv_offload: bad arguments");
  *n_host_evicted = 0;
  if (c->host_pages < 0) return fail(HSTU_ERR_INVALID, "kv_offload: no host tier attached");
  if (!distinct(users, n)) return fail(HSTU_ERR_INVALID, "kv_offload: duplicate users");
  int64_t need = 0;
  for (int32_t b = 0; b < n; ++b) {
    auto it = c->users.find(users[b]);
    if (it == c->users.end()) return fail(HSTU_ERR_UNKNOWN_USER, "kv_offload: user not on the device");
    need += static_cast<int64_t>(it->second.pages.size());
  }
  // room on the host: drop unpinned host users in (tick, id) order
  int64_t have = static_cast<int64_t>(c->host_free_q.size());
  std::vector<std::pair<int64_t, int64_t>> order;
  if (have < need) {
    std::vector<int64_t> pin(pinned, pinned + n_pinned);
    std::sort(pin.begin(), pin.end());
    for (const auto& kv : c->host_users)
      if (!std::binary_search(pin.begin(), pin.end(), kv.first)) order.emplace_back(kv.second.tick, kv.first);
    std::sort(order.begin(), order.end());
  }
  size_t drop = 0;
  while (have < need && drop < order.size()) have += c->host_users.at(order[drop++].second).pages.size();
  if (have < need) return fail(HSTU_ERR_NO_SPACE, "kv_offload: the host tier is too small");
  if (static_cast<int64_t>(drop) > cap) return fail(HSTU_ERR_INVALID, "kv_offload: cap too small");
  std::vector<hstu::PagePair> pairs;
  pairs.reserve(static_cast<size_t>(need));
  for (size_t k = 0; k < drop; ++k) {
    auto it = c->host_users.find(order[k].second);
    for (int32_t pg : it->second.pages) c->host_free_q.push_back(pg);
    host_evicted[k] = it->first;
    c->host_users.erase(it);
  }
  *n_host_evicted = static_cast<int32_t>(drop);
  for (int32_t b = 0; b < n; ++b) {
    auto it = c->users.find(users[b]);
    hstu_kv_cache::User hu;
    hu.len = it->second.len;
    hu.tick = it->second.tick;
    for (int32_t pg : it->second.pages) {
      hu.pages.push_back(c->host_free_q.front());
      c->host_free_q.pop_front();
      pairs.push_back(hstu::PagePair{pg, hu.pages.back()});
      c->free_q.push_back(pg);
    }
    c->host_users.emplace(it->first, std::move(hu));
    c->users.erase(it);
  }
  if (!c->k_pool || pairs.empty()) return ok();
  CopyCtx x{static_cast<int32_t>(pairs.size()), c->num_layers, c->k_pool, c->v_pool, c->num_pages,
            c->host_k, c->host_v, c->host_pages, page_bytes(c), stream};
  return hstu::staged_host(pairs.data(), pairs.size() * sizeof(hstu::PagePair), stream, launch_copy, &x);
}

hstu_status kv_onboard(hstu_kv_cache* c, const int64_t* users, int32_t n, hipStream_t stream) {
  if (!c || n < 0 || (n > 0 && !users)) return fail(HSTU_ERR_INVALID, "kv_onboard: bad arguments");
  if (c->host_pages < 0) return fail(HSTU_ERR_INVALID, "kv_onboard: no host tier attached");
  if (!distinct(users, n)) return fail(HSTU_ERR_INVALID, "kv_onboard: duplicate users");
  int64_t need = 0;
  for (int32_t b = 0; b < n; ++b) {
    auto it = c->host_users.find(users[b]);
    if (it == c->host_users.end()) return fail(HSTU_ERR_UNKNOWN_USER, "kv_onboard: user not on the host tier");
    need += static_cast<int64_t>(it->second.pages.size());
  }
  if (need > static_cast<int64_t>(c->free_q.size()))
    return fail(HSTU_ERR_NO_SPACE, "kv_onboard: not enough free device pages");
  std::vector<hstu::PagePair> pairs;
  pairs.reserve(static_cast<size_t>(need));
  for (int32_t b = 0; b < n; ++b) {
    auto it = c->host_users.find(users[b]);
    hstu_kv_cache::User du;
    du.len = it->second.len;
    du.tick = ++c->tick;
    for (int32_t hp : it->second.pages) {
      du.pages.push_back(c->free_q.front());
      c->free_q.pop_front();
      pairs.push_back(hstu::PagePair{hp, du.pages.back()});
      c->host_free_q.push_back(hp);
    }
    c->users.emplace(it->first, std::move(du));
    c->host_users.erase(it);
  }
  if (!c->k_pool || pairs.empty()) return ok();
  CopyCtx x{static_cast<int32_t>(pairs.size()), c->num_layers, c->host_k, c->host_v, c->host_pages,
            c->k_pool, c->v_pool, c->num_pages, page_bytes(c), stream};
  return hstu::staged_host(pairs.data(), pairs.size() * sizeof(hstu::PagePair), stream, launch_copy, &x);
}

}  // extern "C"

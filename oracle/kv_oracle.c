/*
 * CPU oracle of the paged KV-cache metadata: lookup, allocation, LRU
 * eviction, truncation, the host tier (offload and onboard) and a canonical
 * state dump.
 *
 * TEST INFRASTRUCTURE ONLY (see hstu_oracle.c).  Written independently of the
 * library's manager; the two must produce byte-equal dumps.
 *
 * Source: "Deploying an HSTU Generative Recommender with NVIDIA Dynamo-Triton"
 * (the KVCacheManager paragraph: a paged KV data table in GPU memory with
 * lookup, allocation, append and eviction; older users evicted LRU-style when
 * space is tight).  The pages leave the exact policy open; this follows the
 * plainest reading:
 *   - free pages form a FIFO queue, initially the given order;
 *   - allocation pops from the head; users are served in batch order; a
 *     user's last partial page is filled before a new page is taken, so a user
 *     of length L owns exactly ceil(L / P) pages;
 *   - every user touched by lookup (when present) or allocation gets a fresh
 *     tick from a global counter (pre-incremented), in batch order;
 *   - eviction removes whole users, least tick first (ties: lower id), never a
 *     pinned user, until the free count reaches the request; their pages go to
 *     the tail of the queue in logical order; if the request cannot be met
 *     nothing changes and NO_SPACE is returned;
 *   - truncation frees the whole pages past the new length (tail, logical order);
 *   - allocation and eviction are all-or-nothing.
 * Host tier (same pages: the table spans GPU and host storage, users are
 * onboarded from and offloaded to it):
 *   - a second FIFO queue of host pages, initially 0, 1, 2, ...;
 *   - offload moves device users to the host: if host pages are short, host
 *     users are dropped least tick first (ties: lower id) until enough, their
 *     pages to the host queue's tail in logical order; then, users in order,
 *     each takes host pages from the host queue's head and gives its device
 *     pages to the device queue's tail; length and tick are kept;
 *   - onboard moves host users back: device pages from the device queue's
 *     head, host pages to the host queue's tail, a fresh tick each;
 *   - a host user is absent for lookup and cannot be allocated;
 *   - offload and onboard are all-or-nothing.
 *
 * Canonical dump (little endian, no padding):
 *   u32 magic 0x564B5348, u32 version 1, i32 num_pages, i32 page_size,
 *   i64 tick, i32 n_users, i32 n_free,
 *   per user in ascending id: i64 id, i32 len, i64 tick, i32 n_pages, i32 pages[n_pages]
 *   i32 free[n_free] from head to tail.
 * With a host tier the version is 2 and the dump continues with i32
 * host_pages, i32 n_host_users, i32 n_host_free, the host users in the same
 * form (ascending id) and the host queue from head to tail.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OK 0
#define ERR_INVALID 1
#define ERR_NO_SPACE 2
#define ERR_UNKNOWN_USER 3

typedef struct {
  int64_t id;
  int32_t len;
  int64_t tick;
  int32_t n_pages;
  int32_t *pages; /* capacity num_pages */
} ouser;

typedef struct {
  int32_t num_pages, page_size;
  int64_t tick;
  int32_t *fq; /* ring buffer, capacity num_pages */
  int32_t fq_head, fq_count;
  ouser *users;
  int32_t n_users, cap_users;
  /* host tier (host_pages < 0: none) */
  int32_t host_pages;
  int32_t *hq; /* ring buffer, capacity host_pages */
  int32_t hq_head, hq_count;
  ouser *hosts;
  int32_t n_hosts, cap_hosts;
} oracle_kv;

static int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

oracle_kv *oracle_kv_create(int32_t num_pages, int32_t page_size, const int32_t *free_order) {
  if (num_pages < 0 || page_size <= 0) return NULL;
  oracle_kv *c = (oracle_kv *)calloc(1, sizeof(oracle_kv));
  c->num_pages = num_pages;
  c->page_size = page_size;
  c->fq = (int32_t *)malloc(sizeof(int32_t) * (size_t)(num_pages + 1));
  c->cap_users = 16;
  c->users = (ouser *)calloc((size_t)c->cap_users, sizeof(ouser));
  for (int32_t i = 0; i < num_pages; ++i) c->fq[i] = free_order ? free_order[i] : i;
  c->fq_count = num_pages;
  c->host_pages = -1;
  return c;
}

void oracle_kv_destroy(oracle_kv *c) {
  if (!c) return;
  for (int32_t i = 0; i < c->n_users; ++i) free(c->users[i].pages);
  free(c->users);
  free(c->fq);
  for (int32_t i = 0; i < c->n_hosts; ++i) free(c->hosts[i].pages);
  free(c->hosts);
  free(c->hq);
  free(c);
}

static int find_user(const oracle_kv *c, int64_t id) {
  for (int32_t i = 0; i < c->n_users; ++i)
    if (c->users[i].id == id) return i;
  return -1;
}

static int has_duplicates(const int64_t *ids, int32_t n) {
  for (int32_t a = 0; a < n; ++a)
    for (int32_t b = a + 1; b < n; ++b)
      if (ids[a] == ids[b]) return 1;
  return 0;
}

static void push_free(oracle_kv *c, int32_t page) {
  c->fq[(c->fq_head + c->fq_count) % (c->num_pages ? c->num_pages : 1)] = page;
  c->fq_count++;
}

static int32_t pop_free(oracle_kv *c) {
  int32_t p = c->fq[c->fq_head];
  c->fq_head = (c->fq_head + 1) % c->num_pages;
  c->fq_count--;
  return p;
}

static void remove_user(oracle_kv *c, int idx) {
  ouser *u = &c->users[idx];
  for (int32_t k = 0; k < u->n_pages; ++k) push_free(c, u->pages[k]);
  free(u->pages);
  c->users[idx] = c->users[c->n_users - 1];
  c->n_users--;
}

int oracle_kv_lookup(oracle_kv *c, const int64_t *ids, int32_t B, int32_t *cached_len) {
  if (!c || B < 0 || (B > 0 && (!ids || !cached_len))) return ERR_INVALID;
  if (has_duplicates(ids, B)) return ERR_INVALID;
  for (int32_t b = 0; b < B; ++b) {
    int idx = find_user(c, ids[b]);
    if (idx < 0) {
      cached_len[b] = 0;
    } else {
      cached_len[b] = c->users[idx].len;
      c->users[idx].tick = ++c->tick;
    }
  }
  return OK;
}

/* The LRU choice of users to evict; with drop == 0 it only reports them. */
static int lru_choice(oracle_kv *c, int32_t pages_needed, const int64_t *pinned, int32_t n_pinned,
                      int64_t *evicted, int32_t cap, int32_t *n_evicted, int drop);

int oracle_kv_evict_lru(oracle_kv *c, int32_t pages_needed, const int64_t *pinned, int32_t n_pinned,
                        int64_t *evicted, int32_t cap, int32_t *n_evicted) {
  return lru_choice(c, pages_needed, pinned, n_pinned, evicted, cap, n_evicted, 1);
}

int oracle_kv_lru_victims(oracle_kv *c, int32_t pages_needed, const int64_t *pinned, int32_t n_pinned,
                          int64_t *victims, int32_t cap, int32_t *n_victims) {
  return lru_choice(c, pages_needed, pinned, n_pinned, victims, cap, n_victims, 0);
}

static int lru_choice(oracle_kv *c, int32_t pages_needed, const int64_t *pinned, int32_t n_pinned,
                      int64_t *evicted, int32_t cap, int32_t *n_evicted, int drop) {
  if (!c || pages_needed < 0 || n_pinned < 0 || cap < 0 || !n_evicted) return ERR_INVALID;
  *n_evicted = 0;
  if (c->fq_count >= pages_needed) return OK;
  /* candidates in (tick, id) order, by repeated selection of the minimum */
  int32_t n = c->n_users;
  char *taken = (char *)calloc((size_t)n + 1, 1);
  int *order = (int *)malloc(sizeof(int) * ((size_t)n + 1));
  int32_t n_order = 0;
  int64_t have = c->fq_count;
  while (have < pages_needed) {
    int best = -1;
    for (int32_t i = 0; i < n; ++i) {
      if (taken[i]) continue;
      int pin = 0;
      for (int32_t p = 0; p < n_pinned; ++p)
        if (pinned[p] == c->users[i].id) pin = 1;
      if (pin) continue;
      if (best < 0 || c->users[i].tick < c->users[best].tick ||
          (c->users[i].tick == c->users[best].tick && c->users[i].id < c->users[best].id))
        best = i;
    }
    if (best < 0) break;
    taken[best] = 1;
    order[n_order++] = best;
    have += c->users[best].n_pages;
  }
  int rc = OK;
  if (have < pages_needed) rc = ERR_NO_SPACE;
  else if (n_order > cap) rc = ERR_INVALID;
  if (rc == OK) {
    int64_t *ids = (int64_t *)malloc(sizeof(int64_t) * ((size_t)n_order + 1));
    for (int32_t k = 0; k < n_order; ++k) ids[k] = c->users[order[k]].id;
    for (int32_t k = 0; k < n_order; ++k) {
      if (drop) remove_user(c, find_user(c, ids[k]));
      evicted[k] = ids[k];
    }
    *n_evicted = n_order;
    free(ids);
  }
  free(taken);
  free(order);
  return rc;
}

int oracle_kv_alloc(oracle_kv *c, const int64_t *ids, const int32_t *n_new, int32_t B,
                    int32_t *page_table, int32_t max_pages, int32_t *kv_len) {
  if (!c || B < 0 || max_pages < 0) return ERR_INVALID;
  if (B > 0 && (!ids || !n_new || !kv_len || (max_pages > 0 && !page_table))) return ERR_INVALID;
  if (has_duplicates(ids, B)) return ERR_INVALID;
  int64_t need = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (n_new[b] < 0) return ERR_INVALID;
    for (int32_t h = 0; h < c->n_hosts; ++h)
      if (c->hosts[h].id == ids[b]) return ERR_INVALID; /* onboard first */
    int idx = find_user(c, ids[b]);
    int64_t len = idx < 0 ? 0 : c->users[idx].len;
    int64_t after = len + n_new[b];
    if (after > INT32_MAX) return ERR_INVALID;
    if (ceil_div(after, c->page_size) > max_pages) return ERR_INVALID;
    need += ceil_div(after, c->page_size) - ceil_div(len, c->page_size);
  }
  if (need > c->fq_count) return ERR_NO_SPACE;
  for (int32_t b = 0; b < B; ++b) {
    int idx = find_user(c, ids[b]);
    if (idx < 0) {
      if (c->n_users == c->cap_users) {
        c->cap_users *= 2;
        c->users = (ouser *)realloc(c->users, sizeof(ouser) * (size_t)c->cap_users);
      }
      idx = c->n_users++;
      memset(&c->users[idx], 0, sizeof(ouser));
      c->users[idx].id = ids[b];
      c->users[idx].pages = (int32_t *)malloc(sizeof(int32_t) * (size_t)(c->num_pages + 1));
    }
    ouser *u = &c->users[idx];
    int32_t want = ceil_div((int64_t)u->len + n_new[b], c->page_size);
    while (u->n_pages < want) u->pages[u->n_pages++] = pop_free(c);
    u->len += n_new[b];
    u->tick = ++c->tick;
    kv_len[b] = u->len;
    for (int32_t k = 0; k < max_pages; ++k)
      page_table[(int64_t)b * max_pages + k] = k < u->n_pages ? u->pages[k] : -1;
  }
  return OK;
}

int oracle_kv_truncate(oracle_kv *c, int64_t id, int32_t new_len) {
  if (!c) return ERR_INVALID;
  int idx = find_user(c, id);
  if (idx < 0) return ERR_UNKNOWN_USER;
  ouser *u = &c->users[idx];
  if (new_len < 0 || new_len > u->len) return ERR_INVALID;
  int32_t keep = ceil_div(new_len, c->page_size);
  for (int32_t k = keep; k < u->n_pages; ++k) push_free(c, u->pages[k]);
  u->n_pages = keep;
  u->len = new_len;
  return OK;
}

/* writes the canonical dump; returns its size (buf may be NULL to query) */
int64_t oracle_kv_dump(const oracle_kv *c, uint8_t *buf, int64_t cap) {
  int64_t size = 4 + 4 + 4 + 4 + 8 + 4 + 4;
  for (int32_t i = 0; i < c->n_users; ++i) size += 8 + 4 + 8 + 4 + 4 * (int64_t)c->users[i].n_pages;
  size += 4 * (int64_t)c->fq_count;
  if (c->host_pages >= 0) {
    size += 4 + 4 + 4 + 4 * (int64_t)c->hq_count;
    for (int32_t i = 0; i < c->n_hosts; ++i) size += 8 + 4 + 8 + 4 + 4 * (int64_t)c->hosts[i].n_pages;
  }
  if (!buf || cap < size) return size;
  uint8_t *p = buf;
#define PUT(T, v)                 \
  do {                            \
    T tmp_ = (T)(v);              \
    memcpy(p, &tmp_, sizeof(T));  \
    p += sizeof(T);               \
  } while (0)
  PUT(uint32_t, 0x564B5348u);
  PUT(uint32_t, c->host_pages >= 0 ? 2u : 1u);
  PUT(int32_t, c->num_pages);
  PUT(int32_t, c->page_size);
  PUT(int64_t, c->tick);
  PUT(int32_t, c->n_users);
  PUT(int32_t, c->fq_count);
  /* users in ascending id: selection by the next larger id */
  int64_t last = 0;
  for (int32_t k = 0; k < c->n_users; ++k) {
    int best = -1;
    for (int32_t i = 0; i < c->n_users; ++i) {
      if (k > 0 && c->users[i].id <= last) continue;
      if (best < 0 || c->users[i].id < c->users[best].id) best = i;
    }
    const ouser *u = &c->users[best];
    last = u->id;
    PUT(int64_t, u->id);
    PUT(int32_t, u->len);
    PUT(int64_t, u->tick);
    PUT(int32_t, u->n_pages);
    for (int32_t j = 0; j < u->n_pages; ++j) PUT(int32_t, u->pages[j]);
  }
  for (int32_t k = 0; k < c->fq_count; ++k) PUT(int32_t, c->fq[(c->fq_head + k) % c->num_pages]);
  if (c->host_pages >= 0) {
    PUT(int32_t, c->host_pages);
    PUT(int32_t, c->n_hosts);
    PUT(int32_t, c->hq_count);
    last = 0;
    for (int32_t k = 0; k < c->n_hosts; ++k) {
      int best = -1;
      for (int32_t i = 0; i < c->n_hosts; ++i) {
        if (k > 0 && c->hosts[i].id <= last) continue;
        if (best < 0 || c->hosts[i].id < c->hosts[best].id) best = i;
      }
      const ouser *u = &c->hosts[best];
      last = u->id;
      PUT(int64_t, u->id);
      PUT(int32_t, u->len);
      PUT(int64_t, u->tick);
      PUT(int32_t, u->n_pages);
      for (int32_t j = 0; j < u->n_pages; ++j) PUT(int32_t, u->pages[j]);
    }
    for (int32_t k = 0; k < c->hq_count; ++k) PUT(int32_t, c->hq[(c->hq_head + k) % c->host_pages]);
  }
#undef PUT
  return size;
}

/* ---- host tier ---- */

int oracle_kv_host_attach(oracle_kv *c, int32_t host_pages) {
  if (!c || host_pages < 0 || c->host_pages >= 0) return ERR_INVALID;
  c->host_pages = host_pages;
  c->hq = (int32_t *)malloc(sizeof(int32_t) * (size_t)(host_pages + 1));
  for (int32_t i = 0; i < host_pages; ++i) c->hq[i] = i;
  c->hq_head = 0;
  c->hq_count = host_pages;
  c->cap_hosts = 16;
  c->hosts = (ouser *)calloc((size_t)c->cap_hosts, sizeof(ouser));
  return OK;
}

static void host_push(oracle_kv *c, int32_t page) {
  c->hq[(c->hq_head + c->hq_count) % (c->host_pages ? c->host_pages : 1)] = page;
  c->hq_count++;
}

static int32_t host_pop(oracle_kv *c) {
  int32_t p = c->hq[c->hq_head];
  c->hq_head = (c->hq_head + 1) % c->host_pages;
  c->hq_count--;
  return p;
}

static int find_host(const oracle_kv *c, int64_t id) {
  for (int32_t i = 0; i < c->n_hosts; ++i)
    if (c->hosts[i].id == id) return i;
  return -1;
}

/* where[b]: 0 absent, 1 device, 2 host */
int oracle_kv_residency(const oracle_kv *c, const int64_t *ids, int32_t B, int32_t *where, int32_t *len) {
  if (!c || B < 0) return ERR_INVALID;
  for (int32_t b = 0; b < B; ++b) {
    int d = find_user(c, ids[b]);
    int h = c->host_pages >= 0 ? find_host(c, ids[b]) : -1;
    where[b] = d >= 0 ? 1 : (h >= 0 ? 2 : 0);
    len[b] = d >= 0 ? c->users[d].len : (h >= 0 ? c->hosts[h].len : 0);
  }
  return OK;
}

int oracle_kv_offload(oracle_kv *c, const int64_t *ids, int32_t n, const int64_t *pinned, int32_t n_pinned,
                      int64_t *dropped, int32_t cap, int32_t *n_dropped) {
  if (!c || n < 0 || n_pinned < 0 || cap < 0 || !n_dropped) return ERR_INVALID;
  *n_dropped = 0;
  if (c->host_pages < 0 || has_duplicates(ids, n)) return ERR_INVALID;
  int64_t need = 0;
  for (int32_t b = 0; b < n; ++b) {
    int d = find_user(c, ids[b]);
    if (d < 0) return ERR_UNKNOWN_USER;
    need += c->users[d].n_pages;
  }
  /* unpinned host users to drop, least (tick, id) first */
  char *taken = (char *)calloc((size_t)c->n_hosts + 1, 1);
  int64_t *drop = (int64_t *)malloc(sizeof(int64_t) * ((size_t)c->n_hosts + 1));
  int32_t nd = 0;
  int64_t have = c->hq_count;
  while (have < need) {
    int best = -1;
    for (int32_t i = 0; i < c->n_hosts; ++i) {
      if (taken[i]) continue;
      int pin = 0;
      for (int32_t p = 0; p < n_pinned; ++p)
        if (pinned[p] == c->hosts[i].id) pin = 1;
      if (pin) continue;
      if (best < 0 || c->hosts[i].tick < c->hosts[best].tick ||
          (c->hosts[i].tick == c->hosts[best].tick && c->hosts[i].id < c->hosts[best].id))
        best = i;
    }
    if (best < 0) break;
    taken[best] = 1;
    drop[nd++] = c->hosts[best].id;
    have += c->hosts[best].n_pages;
  }
  int rc = OK;
  if (have < need) rc = ERR_NO_SPACE;
  else if (nd > cap) rc = ERR_INVALID;
  if (rc == OK) {
    for (int32_t k = 0; k < nd; ++k) {
      int h = find_host(c, drop[k]);
      ouser *u = &c->hosts[h];
      for (int32_t j = 0; j < u->n_pages; ++j) host_push(c, u->pages[j]);
      free(u->pages);
      c->hosts[h] = c->hosts[c->n_hosts - 1];
      c->n_hosts--;
      dropped[k] = drop[k];
    }
    *n_dropped = nd;
    for (int32_t b = 0; b < n; ++b) {
      int d = find_user(c, ids[b]);
      ouser *u = &c->users[d];
      if (c->n_hosts == c->cap_hosts) {
        c->cap_hosts *= 2;
        c->hosts = (ouser *)realloc(c->hosts, sizeof(ouser) * (size_t)c->cap_hosts);
      }
      ouser *hu = &c->hosts[c->n_hosts++];
      hu->id = u->id;
      hu->len = u->len;
      hu->tick = u->tick;
      hu->n_pages = u->n_pages;
      hu->pages = (int32_t *)malloc(sizeof(int32_t) * (size_t)(u->n_pages + 1));
      for (int32_t j = 0; j < u->n_pages; ++j) hu->pages[j] = host_pop(c);
      remove_user(c, d); /* device pages to the device queue's tail, logical order */
    }
  }
  free(taken);
  free(drop);
  return rc;
}

int oracle_kv_onboard(oracle_kv *c, const int64_t *ids, int32_t n) {
  if (!c || n < 0 || c->host_pages < 0 || has_duplicates(ids, n)) return ERR_INVALID;
  int64_t need = 0;
  for (int32_t b = 0; b < n; ++b) {
    int h = find_host(c, ids[b]);
    if (h < 0) return ERR_UNKNOWN_USER;
    need += c->hosts[h].n_pages;
  }
  if (need > c->fq_count) return ERR_NO_SPACE;
  for (int32_t b = 0; b < n; ++b) {
    int h = find_host(c, ids[b]);
    ouser *hu = &c->hosts[h];
    if (c->n_users == c->cap_users) {
      c->cap_users *= 2;
      c->users = (ouser *)realloc(c->users, sizeof(ouser) * (size_t)c->cap_users);
    }
    ouser *u = &c->users[c->n_users++];
    u->id = hu->id;
    u->len = hu->len;
    u->tick = ++c->tick;
    u->n_pages = hu->n_pages;
    u->pages = (int32_t *)malloc(sizeof(int32_t) * (size_t)(c->num_pages + 1));
    for (int32_t j = 0; j < hu->n_pages; ++j) {
      u->pages[j] = pop_free(c);
      host_push(c, hu->pages[j]);
    }
    free(hu->pages);
    c->hosts[h] = c->hosts[c->n_hosts - 1];
    c->n_hosts--;
  }
  return OK;
}

/*
 * hstu.h - C ABI of the MI355X (gfx950) HSTU block forward with a paged KV cache.
 *
 * Sources this interface follows:
 *  [GR]  "How Generative Recommenders Are Redefining RecSys at Scale", section
 *        HSTU: attention aggregation with SiLU-based weighting in place of the
 *        softmax, a relative attention bias, and elementwise gating before the
 *        output projection; per-user sequences of interleaved events.
 *  [DT]  "Deploying an HSTU Generative Recommender with NVIDIA Dynamo-Triton"
 *        (and its French and German renderings), section on the KV cache: a
 *        paged KV data table in GPU memory supporting lookup, allocation,
 *        append and eviction, with older users evicted LRU-style when space is
 *        tight; cache-aware operations for lookup, allocation and appending;
 *        the HSTU attention kernel consumes the cached data directly so stable
 *        history is not recomputed; benchmark details: hidden size 512, 4 heads,
 *        BF16 weights, 3- and 8-layer models, batch 8.
 *
 * One HSTU layer, for the new tokens of each user u (positions c_u .. L_u-1
 * of a sequence whose first c_u positions are already cached):
 *     x^        = LayerNorm(x)                 over d_model, biased variance, no affine
 *     [U|V|Q|K] = SiLU(x^ . W1)                W1 [d_model][4*H*dh], chunks U,V,Q,K in
 *                                              that order, head-major inside a chunk
 *     o_i       = (1/n_u) * sum_{j in M(i)} SiLU(q_i . k_j + rab[b(i - j)]) * v_j   (per head)
 *     g         = LayerNorm(o) * U             over all H*dh values of a token, no affine
 *     y         = x + g . W2                   W2 [H*dh][d_model]
 *   M(i) = { j <= i } when i < L_u - T_u (history), else { j < L_u - T_u } u { i }
 *   (the last T_u positions are candidates: they see the whole history and
 *   themselves, not each other).  b(delta) = min(num_buckets - 1,
 *   floor(4 * log2(1 + delta))), one rab table per layer shared by the heads.
 *
 * Conventions
 *  - Every call returns an hstu_status; no exception crosses the ABI.  On an
 *    error hstu_last_error() (thread-local, valid until the next call on the
 *    same thread) describes it.
 *  - "host" pointers are CPU memory read during the call; "device" pointers
 *    are GPU memory owned by the caller.  The library never allocates device
 *    memory: every device buffer (inputs, outputs, weights, pools, page
 *    tables, plan metadata, workspace) belongs to the caller.
 *  - Device work is enqueued asynchronously on the caller's stream.  Host
 *    metadata calls (kv_*, hstu_plan_*) are synchronous and not thread-safe
 *    per handle; the caller serialises them.
 *  - Element types: HSTU_BF16 (bfloat16 storage, fp32 accumulation) or
 *    HSTU_F32.  Matrices are row-major.
 *  - Sequence positions must stay below 65536; bf16 needs head_dim 128;
 *    fp32 supports head_dim 32, 64 or 128.  Other shapes: HSTU_ERR_UNSUPPORTED.
 */
#ifndef HSTU_H
#define HSTU_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSTU_OK = 0,
  HSTU_ERR_INVALID = 1,      /* bad argument; nothing changed */
  HSTU_ERR_NO_SPACE = 2,     /* not enough free pages; nothing changed */
  HSTU_ERR_UNKNOWN_USER = 3, /* user not in the cache */
  HSTU_ERR_DEVICE = 4,       /* a HIP call or kernel launch failed */
  HSTU_ERR_UNSUPPORTED = 5   /* valid, but a shape the library has no kernel for */
} hstu_status;

typedef enum { HSTU_F32 = 0, HSTU_BF16 = 1 } hstu_dtype;

/* Description of the last error on this thread ("" if none). */
const char *hstu_last_error(void);
/* ABI version of this header (currently 1). */
int32_t hstu_abi_version(void);

/* ======================================================================== */
/* KV cache  [DT]: paged table with lookup, allocation, append, LRU eviction */
/* ======================================================================== */

typedef struct hstu_kv_cache hstu_kv_cache;

typedef struct {
  int32_t num_layers, num_heads, head_dim, page_size, num_pages;
  int32_t dtype;    /* hstu_dtype of the pools */
  /* device, each [num_layers][num_pages][num_heads][page_size][head_dim];
   * both NULL for a metadata-only cache (kv_page_append/gather then fail). */
  void *k_pool;
  void *v_pool;
  /* host, a permutation of 0..num_pages-1 giving the initial free-queue
   * order, or NULL for 0, 1, 2, ... (copied during the call) */
  const int32_t *initial_free_order;
} hstu_kv_cache_desc;

/* Creates the host metadata of a cache over caller-owned pools. */
hstu_status kv_cache_create(const hstu_kv_cache_desc *desc, hstu_kv_cache **out);
hstu_status kv_cache_destroy(hstu_kv_cache *cache);

/* lookup [DT]: cached_len[b] (host out) = positions of users[b] already
 * cached, 0 for a user not in the cache.  Each present user gets a fresh LRU
 * tick (global counter, pre-incremented, batch order).  users: host [B],
 * distinct (duplicates: INVALID). */
hstu_status kv_lookup(hstu_kv_cache *cache, const int64_t *users, int32_t B, int32_t *cached_len);

/* eviction [DT]: if fewer than pages_needed pages are free, evicts whole users
 * in ascending (tick, id) order, never one listed in pinned (host
 * [n_pinned]), until free >= pages_needed.  Freed pages join the tail of the
 * free queue in logical order.  evicted (host out, capacity cap) receives the
 * evicted ids in eviction order, *n_evicted their count.  If the request
 * cannot be met: NO_SPACE, nothing changed; if cap is too small: INVALID,
 * nothing changed. */
hstu_status kv_evict_lru(hstu_kv_cache *cache, int32_t pages_needed, const int64_t *pinned,
                         int32_t n_pinned, int64_t *evicted, int32_t cap, int32_t *n_evicted);

/* The users kv_evict_lru would evict for the same arguments (victims, host
 * out [cap], *n_victims), same errors, but nothing changes: with a host tier
 * attached they are offloaded (kv_offload) instead of dropped. */
hstu_status kv_lru_victims(const hstu_kv_cache *cache, int32_t pages_needed, const int64_t *pinned,
                           int32_t n_pinned, int64_t *victims, int32_t cap, int32_t *n_victims);

/* allocation [DT]: reserves room for n_new[b] (host [B]) more positions of
 * users[b] (host [B], distinct; a user not yet cached is created).  Pages
 * come from the head of the free queue, users in batch order; a user's last
 * partial page is filled first, so a user of length L owns ceil(L/P) pages.
 * Each user gets a fresh tick.  Outputs (host): page_table [B][max_pages]
 * (the user's physical pages in logical order, then -1), kv_len [B] (the new
 * length).  All-or-nothing: NO_SPACE if pages are short, INVALID if a user
 * would need more than max_pages pages; nothing changed in either case. */
hstu_status kv_page_alloc(hstu_kv_cache *cache, const int64_t *users, const int32_t *n_new, int32_t B,
                          int32_t *page_table, int32_t max_pages, int32_t *kv_len);

/* Frees the whole pages of `user` past new_len (0 <= new_len <= length) and
 * sets its length; the tick is unchanged.  UNKNOWN_USER / INVALID otherwise. */
hstu_status kv_truncate(hstu_kv_cache *cache, int64_t user, int32_t new_len);

/* Number of free pages (host out). */
hstu_status kv_free_pages(const hstu_kv_cache *cache, int32_t *n_free);

/* Page table of users (host [B]) as kv_page_alloc would return it, without
 * touching ticks; UNKNOWN_USER if one is absent. */
hstu_status kv_page_table(const hstu_kv_cache *cache, const int64_t *users, int32_t B,
                          int32_t *page_table, int32_t max_pages, int32_t *kv_len);

/* Canonical state bytes (little endian): u32 0x564B5348, u32 version (1, or
 * 2 with a host tier attached), i32 num_pages, i32 page_size, i64 tick, i32
 * n_users, i32 n_free; per device-resident user in ascending id: i64 id, i32
 * len, i64 tick, i32 n_pages, i32 pages[n_pages]; then i32 free[n_free] from
 * head to tail.  Version 2 continues with i32 host_pages, i32 n_host_users,
 * i32 n_host_free, the host-resident users in the same form, and the host
 * free queue.  *needed = size; writes only if cap >= size. */
hstu_status kv_state_dump(const hstu_kv_cache *cache, void *buf, size_t cap, size_t *needed);
/* Replaces the metadata with a dump of a cache of the same geometry (the
 * pools are untouched).  INVALID (nothing changed) if inconsistent. */
hstu_status kv_state_load(hstu_kv_cache *cache, const void *buf, size_t len);

/* ---- host tier [DT: the KV data table spans GPU and host storage; users are
 * onboarded from and offloaded to it] ---- */

/* Attaches a host tier of host_pages pages of the same geometry: pools in
 * caller-owned pinned host memory (hipHostMalloc), each
 * [num_layers][host_pages][num_heads][page_size][head_dim], or both NULL for a
 * metadata-only cache.  Its free queue starts as 0, 1, 2, ...  Once per cache
 * (INVALID otherwise). */
hstu_status kv_host_attach(hstu_kv_cache *cache, void *host_k_pool, void *host_v_pool, int32_t host_pages);

/* where[b] (host out) = 0 absent, 1 on the device, 2 on the host tier; len[b]
 * its length (0 if absent).  Ticks unchanged. */
hstu_status kv_residency(const hstu_kv_cache *cache, const int64_t *users, int32_t B, int32_t *where,
                         int32_t *len);

/* offload [DT]: moves device-resident users (host [n], distinct) to the host
 * tier.  If the host free queue is short, host-resident users not listed in
 * pinned (host [n_pinned]) are dropped in ascending (tick, id) order (their
 * pages join the host queue's tail in logical order; their ids go to
 * host_evicted [cap], in drop order).  Then, users in order, each takes its
 * host pages from the host queue's head, copies of every layer's K and V
 * pages to them are enqueued on `stream`, and its device pages join the
 * device free queue's tail in logical order; length and tick are kept.  Work
 * enqueued later on `stream` may reuse the freed device pages; work on other
 * streams must wait for it.  All-or-nothing: UNKNOWN_USER if one is not on
 * the device, NO_SPACE if the host tier cannot hold them, INVALID if cap is
 * too small. */
hstu_status kv_offload(hstu_kv_cache *cache, const int64_t *users, int32_t n, const int64_t *pinned,
                       int32_t n_pinned, hipStream_t stream, int64_t *host_evicted, int32_t cap,
                       int32_t *n_host_evicted);

/* onboard [DT]: moves host-resident users (host [n], distinct) back to the
 * device: users in order, each takes its device pages from the device free
 * queue's head, copies are enqueued on `stream`, its host pages join the host
 * queue's tail in logical order, and it gets a fresh tick.  No eviction
 * here (evict first).  All-or-nothing: UNKNOWN_USER if one is not on the
 * host tier, NO_SPACE if free device pages are short.  A host-resident user
 * counts as absent for kv_lookup and cannot be allocated until onboarded. */
hstu_status kv_onboard(hstu_kv_cache *cache, const int64_t *users, int32_t n, hipStream_t stream);

/* append [DT]: copies the K and V rows of the new tokens into their pages of
 * `layer`.  User b's new rows are d_new_offsets[b] .. d_new_offsets[b+1]-1
 * (device int32 [B+1]) of k_new / v_new (device, row r at r*row_stride
 * elements, H*dh values head-major); they go to positions d_start_pos[b]
 * (device int32 [B]) onwards, through d_page_table (device int32
 * [B][max_pages]).  n_new_total = d_new_offsets[B] (host copy, sizes the
 * launch).  Byte-exact copy. */
hstu_status kv_page_append(const hstu_kv_cache *cache, int32_t layer, int32_t B,
                           const int32_t *d_new_offsets, const int32_t *d_start_pos,
                           const int32_t *d_page_table, int32_t max_pages, const void *k_new,
                           const void *v_new, int64_t row_stride, int32_t n_new_total,
                           hipStream_t stream);

/* gather [DT, KV cache section: the cached history is read back from the
 * paged table instead of being recomputed]: the read side of
 * kv_page_append, for callers that want a user's cached K/V as contiguous
 * rows (inspection, export, a kernel without page-table addressing; the
 * library's own attention reads the pages in place and does not use it).
 * The pages name lookup, allocation, append and eviction, not a gather by
 * name.  Copies positions 0..d_kv_len[b]-1 of each user from the pages of
 * `layer` to contiguous rows d_out_offsets[b].. of k_out / v_out (device,
 * [n_out_total][H*dh]).  Byte-exact copy. */
hstu_status kv_page_gather(const hstu_kv_cache *cache, int32_t layer, int32_t B,
                           const int32_t *d_page_table, int32_t max_pages, const int32_t *d_kv_len,
                           const int32_t *d_out_offsets, int32_t n_out_total, void *k_out,
                           void *v_out, hipStream_t stream);

/* ======================================================================== */
/* Request plan: the jagged batch of one request, scheduled once on the host */
/* and reused by every layer                                                 */
/* ======================================================================== */

typedef struct hstu_plan hstu_plan;

typedef struct {
  int32_t B, num_heads, head_dim;
  const int32_t *new_len;    /* host [B] t_u >= 0: tokens computed this request */
  const int32_t *cached_len; /* host [B] c_u >= 0: positions already cached (0 without a cache) */
  const int32_t *n_targets;  /* host [B] T_u: the last T_u positions of c_u + t_u are candidates */
  const float *norm_n;       /* host [B] n_u (> 0 where t_u > 0), or NULL for n_u = c_u + t_u */
  /* K/V addressing: page_size > 0 reads keys through a page table of
   * max_pages entries per user; page_size == 0 reads contiguous rows. */
  int32_t page_size, max_pages;
} hstu_batch_desc;

typedef struct {
  int32_t n_new_total;       /* sum t_u */
  int32_t n_work_items;      /* attention blocks launched: work items (query block x head x key
                              * range) plus no-op padding of the XCD-aware order */
  int32_t n_partial_slots;   /* fp32 [128][head_dim] partial tiles */
  int64_t pairs;             /* unmasked (query, key) pairs per head */
  size_t meta_bytes;         /* device bytes hstu_plan_upload needs */
  size_t attn_workspace_bytes;
} hstu_plan_info;

hstu_status hstu_plan_create(const hstu_batch_desc *desc, hstu_plan **out);
hstu_status hstu_plan_destroy(hstu_plan *plan);
hstu_status hstu_plan_get_info(const hstu_plan *plan, hstu_plan_info *info);
/* Copies the schedule to d_meta (device, >= meta_bytes, 256-byte aligned) on
 * `stream`, asynchronously (through pinned staging buffers the library keeps
 * for the life of the process); the plan then refers to d_meta, which must
 * outlive its use. */
hstu_status hstu_plan_upload(hstu_plan *plan, void *d_meta, size_t bytes, hipStream_t stream);
/* The attention work items of a plan in launch order (block b of the grid
 * runs record b), for inspection by tests and measurement tools: each record
 * is int32 [6] = user, head, q-block (index in batch order of the blocks of
 * up to 128 new tokens of one user), first and end key tile (64-key tiles
 * [begin, end) of the user's positions), partial slot; slot -1 marks a no-op
 * padding block.  Copies min(n_work_items, cap) records to out (host int32
 * [cap][6]; may be NULL when cap == 0) and sets *n = n_work_items. */
hstu_status hstu_plan_get_items(const hstu_plan *plan, int32_t *out, int32_t cap, int32_t *n);

/* ======================================================================== */
/* Attention [GR]: o = (1/n) sum SiLU(q.k + rab) v over the mask             */
/* ======================================================================== */

typedef struct {
  int32_t dtype;            /* hstu_dtype of q, k, v */
  const hstu_plan *plan;    /* uploaded */
  /* device: query row r (= new token r of the jagged batch) head h at
   * q + r*q_row_stride + h*head_dim */
  const void *q;
  int64_t q_row_stride;
  /* contiguous keys (plan page_size == 0): user u position j is row
   * sum_{w<u}(c_w + t_w) + j of k and v (row stride kv_row_stride) */
  const void *k, *v;
  int64_t kv_row_stride;
  /* paged keys (plan page_size > 0): the cache's pools at `layer`, through
   * d_page_table (device int32 [B][max_pages]); must already hold every
   * position 0..c_u+t_u-1 (append first) */
  const hstu_kv_cache *cache;
  int32_t layer;
  const int32_t *d_page_table;
  const float *rab;         /* device fp32 [num_buckets] */
  int32_t num_buckets;
  float *out;               /* device fp32 [n_new_total][H*head_dim] */
  void *workspace;          /* device, >= attn_workspace_bytes, 256-aligned */
  size_t workspace_bytes;
} hstu_attn_args;

hstu_status hstu_attn_fwd(const hstu_attn_args *args, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, hosts that forbid allocation): hstu_attn_fwd
 * with its fp32 partial tiles in a static device array the library owns, so
 * args->workspace and workspace_bytes are ignored.  Same kernels and the same
 * results as hstu_attn_fwd.  The array holds hstu_attn_static_scratch_bytes()
 * bytes (128 MiB: 2048 partial tiles at head_dim 128); a plan whose
 * attn_workspace_bytes is larger gets HSTU_ERR_UNSUPPORTED with nothing
 * launched.  Every GPU the library runs on keeps its own copy until the
 * process ends; its address is looked up on the first call on that device
 * (with the device current).  Calls on one device share the array: calls
 * that overlap on one device (several streams or host threads) race on it
 * and must be serialised by the caller.  No device or host memory is
 * allocated by this call. */
hstu_status hstu_attn_fwd_static(const hstu_attn_args *args, hipStream_t stream);
size_t hstu_attn_static_scratch_bytes(void);

/* ======================================================================== */
/* One HSTU layer [GR]: pre-norm, f1 + SiLU, (append), attention,            */
/* LayerNorm(o) * U, f2 + residual                                           */
/* ======================================================================== */

typedef struct {
  int32_t dtype;            /* hstu_dtype of x, y, w1, w2, and the pools */
  int32_t d_model;          /* multiple of 128 (bf16) or 4 (fp32) */
  float eps;                /* both LayerNorms */
  const hstu_plan *plan;    /* uploaded */
  const void *x;            /* device [n_new_total][d_model] */
  void *y;                  /* device [n_new_total][d_model], must not overlap x */
  /* weights, output-major (row j holds the inputs' weights of output j):
   * w1 [4*H*head_dim][d_model] is the transpose of the W1 in x . W1, w2
   * [d_model][H*head_dim] the transpose of the W2 in g . W2 */
  const void *w1;
  const void *w2;
  const float *rab;         /* device fp32 [num_buckets] */
  int32_t num_buckets;
  /* paged (plan page_size > 0): K/V of the new tokens are appended to
   * `cache` at `layer` and the attention reads every key from the pages.
   * Contiguous (page_size == 0): every c_u must be 0. */
  const hstu_kv_cache *cache;
  int32_t layer;
  const int32_t *d_page_table;
  void *workspace;          /* device, >= hstu_layer_workspace_size, 256-aligned */
  size_t workspace_bytes;
  /* optional device taps (NULL = skip): [U|V|Q|K] after SiLU
   * [n_new_total][4*H*dh] (dtype), o [n_new_total][H*dh] fp32, g (dtype) */
  void *uvqk_out;
  float *o_out;
  void *g_out;
  /* optional device tap (bf16 only, NULL = skip): the pre-activation
   * LayerNorm(x) . W1 [n_new_total][4*H*dh], which the backward needs */
  void *s_out;
  /* optional (bf16): W1's column sums from hstu_w1_colsum for these weights
   * (device fp32 [4*H*dh]); NULL: computed in every call */
  const float *w1_colsum;
  /* optional (bf16, d_model <= 512): row statistics of a stack's
   * activations, so that a layer's pre-norm needs no pass of its own over x.
   * Layout: device fp32 [n_new_total][d_model/128][2]; entry (r, t) holds the
   * mean and the sum of squared deviations from it of row r's columns
   * 128 t .. 128 t + 127, as stored (bf16-rounded).  y_stats (NULL = skip)
   * receives those of y; x_stats (NULL: this call computes them) must hold
   * those of x, as the previous layer's y_stats does.  Neither may overlap
   * x, y or the workspace. */
  const float *x_stats;
  float *y_stats;
  /* optional (bf16, paged plan): device int64 [n_new_total], where each
   * new-token row's K/V go within one layer of the pools (the element offset
   * of its (page, head 0, slot); -1: not appended).  The same for every
   * layer of one request: a call without x_stats writes it, a call with
   * x_stats on a paged plan requires it and reads it (so the page table must
   * not change between the layers of a request). */
  int64_t *row_slots;
} hstu_layer_args;

/* The column sums of W1 that the bf16 layer's fused pre-norm uses (the sum
 * over d_model of each output column), computed once per weight set: w1 as
 * in hstu_layer_args (device bf16 [rows][d_model], rows = 4*H*dh), out device
 * fp32 [rows].  The values equal those a call without them computes. */
hstu_status hstu_w1_colsum(const void *w1, int32_t rows, int32_t d_model, float *out, hipStream_t stream);

hstu_status hstu_layer_workspace_size(const hstu_layer_args *args, size_t *bytes);
hstu_status hstu_layer_forward(const hstu_layer_args *args, hipStream_t stream);

/* The multi-layer stack [DT: 3- and 8-layer models]: hstu_layer_forward on
 * layers[0..n-1] in order, in one call.  The caller chains the buffers (y of
 * layer i is x of layer i+1; all layers share the plan).  Stops at the first
 * failing layer and returns its status (the message names the layer). */
hstu_status hstu_stack_forward(const hstu_layer_args *layers, int32_t n, hipStream_t stream);

/* ======================================================================== */
/* Backward of one layer, for training ["How Generative Recommenders Are    */
/* Redefining RecSys at Scale", section HSTU support: training of HSTU]      */
/* ======================================================================== */

/* Gradients of a loss L with respect to the layer's input and parameters,
 * given dL/dY, by the chain rule through the layer equations above.  Every
 * position is computed (no cache): the plan is contiguous (page_size 0, every
 * c_u = 0).  bf16 only; head_dim 128, H*head_dim <= 512.  The forward pass
 * supplies what the backward reuses, through hstu_layer_forward's taps:
 * uvqk_out (SiLU'd [U|V|Q|K]), s_out (the pre-activation) and o_out.
 * Activation gradients are bf16, weight and bias gradients fp32.  Every sum
 * runs in a fixed order (no float atomics), so repeated calls give
 * bit-identical gradients. */
typedef struct {
  hstu_dtype dtype;          /* HSTU_BF16 */
  int32_t d_model;           /* multiple of 128, <= 2048 */
  float eps;                 /* the forward's LayerNorm epsilon */
  const hstu_plan *plan;     /* uploaded, contiguous */
  const void *x;             /* device [n][d_model]: the layer's input */
  /* W1 [d_model][4*H*dh] and W2 [H*dh][d_model] in the layout of x . W1 and
   * g . W2 (the transposes of hstu_layer_args' w1 and w2), bf16 */
  const void *w1t;
  const void *w2t;
  const float *rab;          /* device fp32 [num_buckets] (<= 256) */
  int32_t num_buckets;
  const void *uvqk;          /* forward taps: [n][4*H*dh] bf16 */
  const void *s;             /*               [n][4*H*dh] bf16 */
  const float *o;            /*               [n][H*dh] fp32 */
  const void *dy;            /* device [n][d_model] bf16: dL/dY */
  void *dx;                  /* device out [n][d_model] bf16 */
  /* device out fp32, in hstu_layer_args' layouts: dw1 [4*H*dh][d_model],
   * dw2 [d_model][H*dh]; drab [num_buckets] */
  float *dw1;
  float *dw2;
  float *drab;
  void *workspace;           /* device, >= hstu_layer_backward_workspace_size, 256-aligned */
  size_t workspace_bytes;
} hstu_layer_bwd_args;

hstu_status hstu_layer_backward_workspace_size(const hstu_layer_bwd_args *args, size_t *bytes);
/* Enqueues the backward on `stream`.  INVALID for bad arguments, UNSUPPORTED
 * for a paged plan, cached positions, fp32 or unsupported sizes. */
hstu_status hstu_layer_backward(const hstu_layer_bwd_args *args, hipStream_t stream);

/* ======================================================================== */
/* Multitask ranking head ["NVIDIA Dynamo-Triton Gets End-to-End HSTU       */
/* Generative Recommender Workflow", section Recommendation as sequence     */
/* modeling: a prediction head on the HSTU blocks' output gives multitask   */
/* ranking outputs]                                                          */
/* ======================================================================== */

/* The pages name neither the tasks nor the head's shape.  Here, for each
 * listed row y (a row of the last layer's output, normally a candidate's)
 * and each task t, a two-layer perceptron gives the task's logit:
 *     logit[r][t] = b_out[t] + sum_j w_out[t][j] * ReLU(b_hidden[t][j] + y . A_t[:, j])
 * (A_t: task t's [d_model][hidden] first-layer weights).  bf16 MFMA with fp32
 * accumulation; bias, output weights and logits fp32. */
typedef struct {
  hstu_dtype dtype;          /* HSTU_BF16 (HSTU_F32: UNSUPPORTED) */
  int32_t d_model;           /* multiple of 64 */
  int32_t num_tasks;         /* >= 1 */
  int32_t hidden;            /* per task, a multiple of 128 */
  const void *y;             /* device [y_rows][d_model] dtype, rows contiguous, 16-byte aligned */
  int32_t y_rows;
  const int32_t *d_rows;     /* device int32 [n_rows]: rows of y to score (clamped to [0, y_rows)) */
  int32_t n_rows;
  /* weights, output-major: row t*hidden + j of w_hidden [num_tasks*hidden][d_model]
   * (dtype) is A_t[:, j]; b_hidden, w_out fp32 [num_tasks*hidden] (task-major);
   * b_out fp32 [num_tasks].  Device, 16-byte aligned. */
  const void *w_hidden;
  const float *b_hidden;
  const float *w_out;
  const float *b_out;
  float *logits;             /* device out fp32 [n_rows][num_tasks] */
  void *workspace;           /* device, >= hstu_head_workspace_size */
  size_t workspace_bytes;
} hstu_head_args;

hstu_status hstu_head_workspace_size(const hstu_head_args *args, size_t *bytes);
/* Enqueues the head on `stream` (n_rows == 0: nothing).  INVALID for bad
 * sizes or NULL buffers, UNSUPPORTED for fp32. */
hstu_status hstu_head_forward(const hstu_head_args *args, hipStream_t stream);

/* ======================================================================== */
/* Dynamic request batcher ["NVIDIA Dynamo-Triton Gets End-to-End HSTU      */
/* Generative Recommender Workflow", section Five stages and the benchmark: */
/* serving at dynamic batch size 8; "HSTU生成式推荐系统部署实战：NVIDIA      */
/* Dynamo-Triton详解", Triton section: dynamic batching]                     */
/* ======================================================================== */

/* Host-only request queue.  A request is (request_id, user, n_new tokens,
 * arrival time in microseconds on the caller's clock).  The next batch is
 * read off the queue in submission order, skipping a request whose user is
 * already in the batch (the KV cache takes each user once per request) and
 * stopping at max_batch requests or before the first request that would take
 * the batch past max_tokens new tokens (0: no limit; a first request is always
 * taken).  The batch is released when no further request can join it (full)
 * or when the oldest queued request has waited max_delay_us. */
typedef struct hstu_batcher hstu_batcher;
typedef struct {
  int32_t max_batch;     /* >= 1 */
  int64_t max_delay_us;  /* >= 0 */
  int64_t max_tokens;    /* >= 0, 0 = no token budget */
} hstu_batcher_desc;

hstu_status hstu_batcher_create(const hstu_batcher_desc *desc, hstu_batcher **out);
hstu_status hstu_batcher_destroy(hstu_batcher *batcher);
/* Queues one request (n_new >= 0). */
hstu_status hstu_batcher_submit(hstu_batcher *batcher, int64_t request_id, int64_t user, int32_t n_new,
                                int64_t arrival_us);
/* At time now_us: if a batch is released, its request ids (host out, capacity
 * cap, batch order = submission order) and *n = its size, *wait_us = 0; they
 * leave the queue.  Otherwise *n = 0 and *wait_us = the time until the oldest
 * request's delay runs out (-1: queue empty).  INVALID (queue unchanged) if
 * cap is smaller than the released batch. */
hstu_status hstu_batcher_next(hstu_batcher *batcher, int64_t now_us, int64_t *request_ids, int32_t cap,
                              int32_t *n, int64_t *wait_us);
/* *n = queued requests. */
hstu_status hstu_batcher_pending(const hstu_batcher *batcher, int32_t *n);

/* ======================================================================== */
/* Instrumentation: kernel durations measured with HIP events               */
/* ======================================================================== */

/* When enabled (non-zero), every kernel the library launches is bracketed
 * by a pair of HIP events recorded on the stream it is launched on.  Kernel
 * names: "layer_norm", "f1_gemm", "append", "attention", "reduce_gate",
 * "f2_gemm", "gather", "head", "bwd_attention", "bwd_gemm" (the backward's
 * products), "bwd_rows" (its row and elementwise kernels).  With enable == 2
 * the attention of a request planned while enable == 2 (hstu_plan_create)
 * that mixes users with a cached prefix and users without one runs as two
 * grids, recorded as "attention_cached" (the users
 * with a prefix: few queries against many cached keys) and
 * "attention_prefill" (the rest); other requests record "attention".  The
 * results are the same either way.  Enabling or disabling clears the
 * records. */
hstu_status hstu_timing_enable(int32_t enable);
/* Waits for the recorded events of `kernel` and returns the number of
 * launches and their summed duration in milliseconds; clears them.
 * INVALID for an unknown name. */
hstu_status hstu_timing_read(const char *kernel, int32_t *launches, double *total_ms);

/* Phase records of the bf16 attention: with d_stamps (device, 16-byte
 * aligned) registered for `capacity` records, every later single-grid bf16
 * attention launch of a plan with at most `capacity` blocks writes, for
 * block b, record b (48 bytes): uint64 start, setup_done, loop_done, end
 * (the 100 MHz realtime clock at the block's start, after its set-up, after
 * its key-tile loop, at its end), uint32 hw_id (the HW_ID register: CU in
 * bits 8-11, shader engine in bits 13-14), uint32 xcc_id (the XCD), int32
 * slot and int32 tiles (the work item's partial slot and key-tile range;
 * padding blocks write nothing).  Each launch overwrites the records; the
 * caller reads them after synchronising.  The buffer belongs to the device
 * current at registration; launches on other devices write no records.
 * capacity 0 (d_stamps NULL) switches the records off.  Costs one uniform
 * branch a block when off. */
hstu_status hstu_attn_stamps(void *d_stamps, int64_t capacity);

/* Achievable ceilings of the two resources the layer is bound by (the
 * benchmark quotes roofline fractions against these beside the vendor
 * peaks; the pages state their target as a fraction of the HBM / MFMA
 * roofline).  Each enqueues one kernel on `stream`; time it with events.
 *  hstu_ceiling_mfma: `blocks` blocks of 256 threads, each wave issuing
 *    4 * iters back-to-back bf16 32x32x16 MFMAs (4 * iters * 32768 FLOPs a
 *    wave); `out` (device fp32 [blocks]) is written only in a case that
 *    does not occur, so the launch does no memory traffic.
 *  hstu_ceiling_read: reads `bytes` (multiple of 16, 16-byte aligned) of
 *    device memory once; `out` (device uint32 [4096]) as above.
 *  hstu_ceiling_copy: copies `bytes` from src to dst (device, disjoint).
 * INVALID for null pointers, non-positive sizes or misalignment. */
hstu_status hstu_ceiling_mfma(int32_t blocks, int32_t iters, float *out, hipStream_t stream);
hstu_status hstu_ceiling_read(const void *src, int64_t bytes, void *out, hipStream_t stream);
hstu_status hstu_ceiling_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HSTU_H */

// C ABI of libhstu: error state, the request plan (a host-side schedule of
// the attention work, built once per request and reused by every layer),
// and the drivers of hstu_attn_fwd / hstu_layer_forward / kv_page_append /
// kv_page_gather.  Every arithmetic step runs in the HIP kernels under
// kernels/; this file only validates, schedules and launches.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <numeric>
#include <tuple>

#include "internal.h"

namespace hstu {

namespace {
thread_local std::string g_last_error;
}

hstu_status fail(hstu_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}
hstu_status ok() {
  g_last_error.clear();
  return HSTU_OK;
}
hstu_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return HSTU_OK;
  return fail(HSTU_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

namespace {

template <typename F>
hipError_t timed(TimedKernel k, hipStream_t s, F&& f) {
  TimedLaunch t(k, s);
  hipError_t e = f();
  t.end();
  return e;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
size_t esize(int dtype) { return dtype == HSTU_BF16 ? 2 : 4; }

// Attention work per key tile is roughly constant, so pieces are sized in
// visible tiles.  Enough pieces to give every CU several, but never pieces so
// small that their partial tile costs more than the keys they read.
#ifndef HSTU_TARGET_PIECES  // compile-time tuning knobs (defaults measured best on MI355X)
#define HSTU_TARGET_PIECES 768
#endif
#ifndef HSTU_MIN_PIECE_TILES
#define HSTU_MIN_PIECE_TILES 4
#endif
constexpr int kTargetPieces = HSTU_TARGET_PIECES;
constexpr int kMinPieceTiles = HSTU_MIN_PIECE_TILES;
constexpr int kMaxPieceTiles = 256;  // bounds a work item's staged page-table slice
constexpr int kXcds = 8;             // workgroups are dealt to the 8 XCDs round-robin

// Pinned staging for host-to-device uploads, so they are truly asynchronous
// and the host can plan the next request while the GPU runs this one.  A
// small ring of pinned buffers, each reused only after its previous copy has
// completed (an event recorded behind it); buffers grow on demand and live
// until the process ends.
struct StagingRing {
  struct Slot {
    void* host = nullptr;
    size_t cap = 0;
    hipEvent_t done = nullptr;
    bool pending = false;
  };
  std::mutex mu;
  Slot slots[4];
  int next = 0;
};

StagingRing& staging() {
  static StagingRing r;
  return r;
}


// Dispatch order of attention pieces (visible tiles, item), appended to out.
// Block b runs on XCD b % 8, and each XCD starts its next block as soon as
// one of its slots frees, independently of the others, so the launch ends
// when the most loaded XCD drains.  Pieces of one (user, head) read the same
// K/V and go to one XCD where the balance allows, sharing its L2: groups are
// taken largest first, each onto the least-loaded XCD, and a piece that
// would lift that XCD above an equal share of all tiles goes to the
// least-loaded XCD instead.  Each XCD then runs its pieces longest first
// (ties keep the group order), so that its last slots free together; XCD
// x's k-th piece sits at index 8k + x and short queues are padded with no-op
// entries (slot -1), so out grows by a multiple of 8.
void dispatch_order(const std::vector<std::pair<int32_t, WorkItem>>& pieces, const std::vector<int32_t>& sel,
                    int32_t B, int32_t H, std::vector<WorkItem>& out) {
  // pieces are handled by index (sel: the pieces to order, in input order)
  const int32_t n = static_cast<int32_t>(sel.size());
  auto tiles = [&](int32_t i) { return pieces[i].first; };
  // groups in order of first appearance, each group's pieces in input order
  std::vector<int32_t> gid(static_cast<size_t>(B) * H, -1), gfirst, gcount;
  std::vector<int64_t> gcost;
  std::vector<int32_t> pg(n);
  int64_t all = 0;
  for (int32_t k = 0; k < n; ++k) {
    const WorkItem& w = pieces[sel[k]].second;
    int32_t& g = gid[static_cast<size_t>(w.user) * H + w.head];
    if (g < 0) {
      g = static_cast<int32_t>(gcost.size());
      gcost.push_back(0);
      gcount.push_back(0);
    }
    pg[k] = g;
    gcost[g] += tiles(sel[k]);
    ++gcount[g];
    all += tiles(sel[k]);
  }
  const int32_t ng = static_cast<int32_t>(gcost.size());
  gfirst.assign(ng + 1, 0);
  for (int32_t g = 0; g < ng; ++g) gfirst[g + 1] = gfirst[g] + gcount[g];
  std::vector<int32_t> byg(n), fill(gfirst.begin(), gfirst.end() - 1);
  for (int32_t k = 0; k < n; ++k) byg[fill[pg[k]]++] = sel[k];
  const int64_t share = (all + kXcds - 1) / kXcds;
  // Sorts run on 64-bit keys (visible tiles descending in the high half, the
  // tie-break ascending in the low half): the stable orders, without the
  // temporary buffers of std::stable_sort or indirect compares.
  auto key = [&](int32_t tiles_, int32_t tie) {
    return (static_cast<uint64_t>(static_cast<uint32_t>(INT32_MAX - tiles_)) << 32) | static_cast<uint32_t>(tie);
  };
  std::vector<int32_t> gorder(ng);
  std::iota(gorder.begin(), gorder.end(), 0);
  std::sort(gorder.begin(), gorder.end(),
            [&](int32_t a, int32_t b) { return gcost[a] != gcost[b] ? gcost[a] > gcost[b] : a < b; });
  // per XCD, keys of (visible tiles, assignment order); seq_piece maps the
  // assignment order back to the piece
  std::vector<std::vector<uint64_t>> q(kXcds);
  for (auto& qq : q) qq.reserve(static_cast<size_t>(n) / kXcds + 1);
  std::vector<int32_t> seq_piece;
  seq_piece.reserve(n);
  std::vector<uint64_t> gk;
  std::vector<int64_t> load(kXcds, 0);
  auto least = [&]() { return static_cast<int>(std::min_element(load.begin(), load.end()) - load.begin()); };
  for (int32_t gi : gorder) {
    // a group's pieces, longest first, ties in input order (increasing index)
    gk.clear();
    for (int32_t k = gfirst[gi]; k < gfirst[gi + 1]; ++k) gk.push_back(key(tiles(byg[k]), byg[k]));
    std::sort(gk.begin(), gk.end());
    const int home = least();
    for (uint64_t kv : gk) {
      const int32_t i = static_cast<int32_t>(kv & 0xFFFFFFFFu);
      const int x = load[home] + tiles(i) <= share ? home : least();
      q[x].push_back(key(tiles(i), static_cast<int32_t>(seq_piece.size())));
      seq_piece.push_back(i);
      load[x] += tiles(i);
    }
  }
  size_t depth = 0;
  for (auto& qq : q) {
    std::sort(qq.begin(), qq.end());
    depth = std::max(depth, qq.size());
  }
  WorkItem pad{};
  pad.slot = -1;
  out.reserve(out.size() + depth * kXcds);
  for (size_t k = 0; k < depth; ++k)
    for (int x = 0; x < kXcds; ++x)
      out.push_back(k < q[x].size() ? pieces[seq_piece[q[x][k] & 0xFFFFFFFFu]].second : pad);
}

}  // namespace

namespace {
// Takes the next slot of the ring (waiting for its previous use), sized for
// `bytes`, and fills it from src.  Caller holds the ring's lock.
hstu_status fill_slot(StagingRing& r, const void* src, size_t bytes, StagingRing::Slot** out) {
  StagingRing::Slot& sl = r.slots[r.next];
  r.next = (r.next + 1) % 4;
  hstu_status st;
  if (sl.pending) {
    // poll rather than block: a blocking wait can sleep past the event, and
    // the slot's previous upload is normally long done
    hipError_t q;
    while ((q = hipEventQuery(sl.done)) == hipErrorNotReady) {
    }
    if ((st = check_hip(q, "staging")) != HSTU_OK) return st;
    sl.pending = false;
  }
  if (!sl.done && (st = check_hip(hipEventCreateWithFlags(&sl.done, hipEventDisableTiming), "staging")) != HSTU_OK)
    return st;
  if (sl.cap < bytes) {
    if (sl.host && (st = check_hip(hipHostFree(sl.host), "staging")) != HSTU_OK) return st;
    sl.host = nullptr;
    sl.cap = 0;
    size_t want = std::max(bytes, static_cast<size_t>(1) << 20);
    if ((st = check_hip(hipHostMalloc(&sl.host, want, hipHostMallocDefault), "staging")) != HSTU_OK)
      return st;
    sl.cap = want;
  }
  std::memcpy(sl.host, src, bytes);
  *out = &sl;
  return HSTU_OK;
}
}  // namespace

hstu_status staged_upload(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return HSTU_OK;
  StagingRing& r = staging();
  std::lock_guard<std::mutex> lk(r.mu);
  StagingRing::Slot* sl = nullptr;
  hstu_status st;
  if ((st = fill_slot(r, src, bytes, &sl)) != HSTU_OK) return st;
  if ((st = check_hip(hipMemcpyAsync(dst, sl->host, bytes, hipMemcpyHostToDevice, stream), "staged upload")) !=
      HSTU_OK)
    return st;
  if ((st = check_hip(hipEventRecord(sl->done, stream), "staged upload")) != HSTU_OK) return st;
  sl->pending = true;
  return HSTU_OK;
}

hstu_status staged_host(const void* src, size_t bytes, hipStream_t stream,
                        hipError_t (*use)(const void* slot, void* ctx), void* ctx) {
  if (bytes == 0) return HSTU_OK;
  StagingRing& r = staging();
  std::lock_guard<std::mutex> lk(r.mu);
  StagingRing::Slot* sl = nullptr;
  hstu_status st;
  if ((st = fill_slot(r, src, bytes, &sl)) != HSTU_OK) return st;
  void* dev = nullptr;
  if ((st = check_hip(hipHostGetDevicePointer(&dev, sl->host, 0), "staging")) != HSTU_OK) return st;
  if ((st = check_hip(use(dev, ctx), "staged launch")) != HSTU_OK) return st;
  if ((st = check_hip(hipEventRecord(sl->done, stream), "staging")) != HSTU_OK) return st;
  sl->pending = true;
  return HSTU_OK;
}

// the buffer registered with hstu_attn_stamps
std::mutex g_stamps_mu;
AttnStamp* g_stamps = nullptr;
int64_t g_stamps_cap = 0;
int g_stamps_dev = -1;  // the device current when the buffer was registered

AttnStamp* attn_stamps_for(int32_t n_items) {
  std::lock_guard<std::mutex> lk(g_stamps_mu);
  if (!g_stamps || n_items > g_stamps_cap) return nullptr;
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess && dev == g_stamps_dev ? g_stamps : nullptr;
}

}  // namespace hstu

using namespace hstu;

extern "C" {

const char* hstu_last_error(void) { return g_last_error.c_str(); }
int32_t hstu_abi_version(void) { return 1; }

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

hstu_status hstu_plan_create(const hstu_batch_desc* d, hstu_plan** out) {
  if (!d || !out) return fail(HSTU_ERR_INVALID, "hstu_plan_create: null argument");
  *out = nullptr;
  const int32_t B = d->B, H = d->num_heads, dh = d->head_dim;
  if (B < 0 || H <= 0 || dh <= 0) return fail(HSTU_ERR_INVALID, "hstu_plan_create: bad B/H/dh");
  if (B > 0 && (!d->new_len || !d->cached_len || !d->n_targets))
    return fail(HSTU_ERR_INVALID, "hstu_plan_create: null per-user array");
  if (dh != 32 && dh != 64 && dh != 128)
    return fail(HSTU_ERR_UNSUPPORTED, "hstu_plan_create: head_dim must be 32, 64 or 128");
  if (d->page_size < 0 || (d->page_size > 0 && d->max_pages <= 0))
    return fail(HSTU_ERR_INVALID, "hstu_plan_create: bad page_size/max_pages");
  auto* p = new hstu_plan();
  p->desc = *d;
  p->new_len.assign(d->new_len, d->new_len + B);
  p->cached_len.assign(d->cached_len, d->cached_len + B);
  p->n_targets.assign(d->n_targets, d->n_targets + B);
  p->norm_n.resize(B);
  p->desc.new_len = p->desc.cached_len = p->desc.n_targets = nullptr;
  p->desc.norm_n = nullptr;
  int64_t q_row = 0, kv_row = 0;
  p->new_offsets.push_back(0);
  for (int32_t u = 0; u < B; ++u) {
    int64_t t = p->new_len[u], c = p->cached_len[u], T = p->n_targets[u];
    int64_t L = t + c;
    if (t < 0 || c < 0 || T < 0 || T > L) {
      delete p;
      return fail(HSTU_ERR_INVALID, "hstu_plan_create: bad new_len/cached_len/n_targets");
    }
    if (L > kMaxPos) {
      delete p;
      return fail(HSTU_ERR_UNSUPPORTED, "hstu_plan_create: sequence longer than 65535");
    }
    if (d->page_size > 0 && L > static_cast<int64_t>(d->max_pages) * d->page_size) {
      delete p;
      return fail(HSTU_ERR_INVALID, "hstu_plan_create: max_pages * page_size < sequence length");
    }
    float n = d->norm_n ? d->norm_n[u] : static_cast<float>(L);
    if (t > 0 && (!(n > 0.f) || !std::isfinite(n))) {
      delete p;
      return fail(HSTU_ERR_INVALID, "hstu_plan_create: norm_n must be positive");
    }
    p->norm_n[u] = n;
    UserInfo ui{};
    ui.q_row0 = static_cast<int32_t>(q_row);
    ui.n_new = static_cast<int32_t>(t);
    ui.start = static_cast<int32_t>(c);
    ui.kv_len = static_cast<int32_t>(L);
    ui.hist = static_cast<int32_t>(L - T);
    ui.kv_row0 = static_cast<int32_t>(kv_row);
    ui.inv_n = t > 0 ? 1.0f / n : 0.0f;
    p->users.push_back(ui);
    p->start_pos.push_back(static_cast<int32_t>(c));
    q_row += t;
    kv_row += L;
    if (q_row > INT32_MAX / 4 || kv_row > INT32_MAX / 4) {
      delete p;
      return fail(HSTU_ERR_UNSUPPORTED, "hstu_plan_create: batch too large");
    }
    p->new_offsets.push_back(static_cast<int32_t>(q_row));
    p->max_len = std::max<int32_t>(p->max_len, static_cast<int32_t>(L));
    // unmasked pairs of this user's new queries
    // (a history query i sees i + 1 keys, a candidate the L - T history keys and itself)
    {
      const int64_t h = L - T, a = c, b = std::min(L, h);
      if (b > a) p->pairs += (b * (b + 1) - a * (a + 1)) / 2;
      const int64_t nc = L - std::max(c, h);
      if (nc > 0) p->pairs += nc * (h + 1);
    }
  }
  p->n_new = static_cast<int32_t>(q_row);

  // q-blocks
  p->row_pos.resize(p->n_new);
  for (int32_t u = 0; u < B; ++u) {
    const UserInfo& ui = p->users[u];
    for (int32_t r = 0; r < ui.n_new; ++r) p->row_pos[ui.q_row0 + r] = RowPos{u, ui.start + r};
    for (int32_t r = 0; r < ui.n_new; r += kBlockQ)
      p->qblocks.push_back(QBlock{u, ui.q_row0 + r, std::min(kBlockQ, ui.n_new - r), ui.start + r});
  }
  // visible key tiles of each q-block, then pieces
  const int32_t nqb = static_cast<int32_t>(p->qblocks.size());
  std::vector<std::vector<int32_t>> vis(nqb);
  int64_t total = 0;
  for (int32_t b = 0; b < nqb; ++b) {
    const QBlock& qb = p->qblocks[b];
    const UserInfo& ui = p->users[qb.user];
    int64_t qa = qb.pos0, qe = qb.pos0 + qb.count;
    // tile_visible as two ranges: the band of tiles holding the block's own
    // positions, [qa / 64, ntiles), and the tiles below min(hist, qe - 1)
    const int32_t ntiles = static_cast<int32_t>((qe + kTileK - 1) / kTileK);
    const int64_t lim = std::min<int64_t>(ui.hist, qe - 1);
    const int32_t lo_end = lim > 0 ? static_cast<int32_t>(std::min<int64_t>((lim + kTileK - 1) / kTileK, ntiles)) : 0;
    const int32_t band = static_cast<int32_t>(qa / kTileK);
    vis[b].reserve(ntiles);
    for (int32_t t = 0; t < lo_end; ++t) vis[b].push_back(t);
    for (int32_t t = std::max(band, lo_end); t < ntiles; ++t) vis[b].push_back(t);
    total += static_cast<int64_t>(vis[b].size()) * H;
  }
  int64_t piece_tiles = std::min<int64_t>(
      kMaxPieceTiles, std::max<int64_t>(kMinPieceTiles, (total + kTargetPieces - 1) / kTargetPieces));
  p->qb_slots.resize(static_cast<size_t>(nqb) * H);
  std::vector<std::pair<int32_t, WorkItem>> pieces;  // (visible tiles, item)
  int32_t slot = 0;
  // page-table entries a paged piece over tiles [tb, te) stages
  const int64_t P = d->page_size;
  auto span_pages = [&](int64_t tb, int64_t te) -> int64_t {
    return P > 0 ? (te * kTileK + P - 1) / P - tb * kTileK / P : 0;
  };
  std::vector<std::pair<int32_t, int32_t>> cuts;  // [lo, hi) into the visible-tile list
  for (int32_t b = 0; b < nqb; ++b) {
    const auto& v = vis[b];
    int32_t nv = static_cast<int32_t>(v.size());
    int32_t np = std::max<int32_t>(1, static_cast<int32_t>((nv + piece_tiles - 1) / piece_tiles));
    // equal shares of the visible tiles, each cut again wherever its page
    // span would pass kMaxItemPages (one tile spans at most 5 pages, P >= 16)
    cuts.clear();
    for (int32_t k = 0; k < np; ++k) {
      int32_t lo = static_cast<int32_t>(static_cast<int64_t>(nv) * k / np);
      int32_t hi = static_cast<int32_t>(static_cast<int64_t>(nv) * (k + 1) / np);
      int32_t start = lo;
      for (int32_t i = lo + 1; i < hi; ++i)
        if (span_pages(v[start], v[i] + 1) > kMaxItemPages) {
          cuts.emplace_back(start, i);
          start = i;
        }
      cuts.emplace_back(start, hi);
    }
    const int32_t npc = static_cast<int32_t>(cuts.size());
    for (int32_t h = 0; h < H; ++h) {
      p->qb_slots[static_cast<size_t>(b) * H + h] = SlotRange{slot, npc};
      for (const auto& cut : cuts) {
        const int32_t lo = cut.first, hi = cut.second;
        const QBlock& qb = p->qblocks[b];
        const UserInfo& ui = p->users[qb.user];
        WorkItem w{};
        w.user = qb.user;
        w.head = h;
        w.qblock = b;
        w.tile_begin = nv ? v[lo] : 0;
        w.tile_end = nv ? v[hi - 1] + 1 : 0;
        w.slot = slot++;
        w.row0 = qb.row0;
        w.count = qb.count;
        w.pos0 = qb.pos0;
        w.kv_len = ui.kv_len;
        w.hist = ui.hist;
        w.kv_row0 = ui.kv_row0;
        pieces.emplace_back(hi - lo, w);
      }
    }
  }
  p->n_slots = slot;
  {
    std::vector<int32_t> sel(pieces.size());
    std::iota(sel.begin(), sel.end(), 0);
    dispatch_order(pieces, sel, B, H, p->items);
  }
  // The same pieces again as two consecutive orders, those of users with a
  // cached prefix first (few queries against a long prefix: the bandwidth
  // regime) and then the others (the full-recompute regime), when a request
  // has both and the plan is made while split timing is on: instrumented
  // runs launch them as two grids to time each.
  if (timing_mode() == 2) {
    std::vector<int32_t> cached_sel, prefill_sel;
    for (int32_t i = 0; i < static_cast<int32_t>(pieces.size()); ++i)
      (p->users[pieces[i].second.user].start > 0 ? cached_sel : prefill_sel).push_back(i);
    if (!cached_sel.empty() && !prefill_sel.empty()) {
      dispatch_order(pieces, cached_sel, B, H, p->items_split);
      p->n_split_cached = static_cast<int32_t>(p->items_split.size());
      dispatch_order(pieces, prefill_sel, B, H, p->items_split);
    }
  }

  // packed device image
  auto& blob = p->host_blob;
  size_t off = 0;
  auto region = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + std::max<size_t>(bytes, 1));
    return o;
  };
  p->off_items = region(p->items.size() * sizeof(WorkItem));
  p->off_items_split = region(p->items_split.size() * sizeof(WorkItem));
  p->off_qblocks = region(p->qblocks.size() * sizeof(QBlock));
  p->off_qb_slots = region(p->qb_slots.size() * sizeof(SlotRange));
  p->off_users = region(p->users.size() * sizeof(UserInfo));
  p->off_row_pos = region(p->row_pos.size() * sizeof(RowPos));
  p->off_new_offsets = region(p->new_offsets.size() * sizeof(int32_t));
  p->off_start_pos = region(p->start_pos.size() * sizeof(int32_t));
  blob.assign(off, 0);
  auto copy = [&](size_t o, const void* src, size_t bytes) {
    if (bytes) std::memcpy(blob.data() + o, src, bytes);
  };
  copy(p->off_items, p->items.data(), p->items.size() * sizeof(WorkItem));
  copy(p->off_items_split, p->items_split.data(), p->items_split.size() * sizeof(WorkItem));
  copy(p->off_qblocks, p->qblocks.data(), p->qblocks.size() * sizeof(QBlock));
  copy(p->off_qb_slots, p->qb_slots.data(), p->qb_slots.size() * sizeof(SlotRange));
  copy(p->off_users, p->users.data(), p->users.size() * sizeof(UserInfo));
  copy(p->off_row_pos, p->row_pos.data(), p->row_pos.size() * sizeof(RowPos));
  copy(p->off_new_offsets, p->new_offsets.data(), p->new_offsets.size() * sizeof(int32_t));
  copy(p->off_start_pos, p->start_pos.data(), p->start_pos.size() * sizeof(int32_t));
  *out = p;
  return ok();
}

hstu_status hstu_plan_destroy(hstu_plan* p) {
  delete p;
  return ok();
}

hstu_status hstu_plan_get_info(const hstu_plan* p, hstu_plan_info* info) {
  if (!p || !info) return fail(HSTU_ERR_INVALID, "hstu_plan_get_info: null argument");
  info->n_new_total = p->n_new;
  info->n_work_items = static_cast<int32_t>(p->items.size());
  info->n_partial_slots = p->n_slots;
  info->pairs = p->pairs;
  info->meta_bytes = p->host_blob.size();
  info->attn_workspace_bytes =
      align256(static_cast<size_t>(p->n_slots) * kBlockQ * p->desc.head_dim * sizeof(float));
  return ok();
}

hstu_status hstu_plan_get_items(const hstu_plan* p, int32_t* out, int32_t cap, int32_t* n) {
  if (!p || !n || cap < 0 || (cap > 0 && !out)) return fail(HSTU_ERR_INVALID, "hstu_plan_get_items: bad argument");
  const int32_t total = static_cast<int32_t>(p->items.size());
  for (int32_t i = 0; i < std::min(total, cap); ++i) {
    const WorkItem& w = p->items[i];
    int32_t* r = out + static_cast<int64_t>(i) * 6;
    r[0] = w.user;
    r[1] = w.head;
    r[2] = w.qblock;
    r[3] = w.tile_begin;
    r[4] = w.tile_end;
    r[5] = w.slot;
  }
  *n = total;
  return ok();
}

hstu_status hstu_plan_upload(hstu_plan* p, void* d_meta, size_t bytes, hipStream_t stream) {
  if (!p || !d_meta) return fail(HSTU_ERR_INVALID, "hstu_plan_upload: null argument");
  if (bytes < p->host_blob.size()) return fail(HSTU_ERR_INVALID, "hstu_plan_upload: buffer too small");
  if (reinterpret_cast<uintptr_t>(d_meta) % 256)
    return fail(HSTU_ERR_INVALID, "hstu_plan_upload: d_meta must be 256-byte aligned");
  hstu_status st = staged_upload(d_meta, p->host_blob.data(), p->host_blob.size(), stream);
  if (st != HSTU_OK) return st;
  auto* base = static_cast<unsigned char*>(d_meta);
  p->d_meta = d_meta;
  PlanDev& dv = p->dev;
  dv.items = reinterpret_cast<const WorkItem*>(base + p->off_items);
  p->d_items_split = reinterpret_cast<const WorkItem*>(base + p->off_items_split);
  dv.qblocks = reinterpret_cast<const QBlock*>(base + p->off_qblocks);
  dv.qb_slots = reinterpret_cast<const SlotRange*>(base + p->off_qb_slots);
  dv.users = reinterpret_cast<const UserInfo*>(base + p->off_users);
  dv.row_pos = reinterpret_cast<const RowPos*>(base + p->off_row_pos);
  dv.new_offsets = reinterpret_cast<const int32_t*>(base + p->off_new_offsets);
  dv.start_pos = reinterpret_cast<const int32_t*>(base + p->off_start_pos);
  dv.n_items = static_cast<int32_t>(p->items.size());
  dv.n_qblocks = static_cast<int32_t>(p->qblocks.size());
  dv.n_new = p->n_new;
  dv.B = p->desc.B;
  dv.H = p->desc.num_heads;
  dv.dh = p->desc.head_dim;
  dv.page_size = p->desc.page_size;
  dv.max_pages = p->desc.max_pages;
  dv.max_len = p->max_len;
  return ok();
}

// ---------------------------------------------------------------------------
// KV data movement
// ---------------------------------------------------------------------------

hstu_status kv_page_append(const hstu_kv_cache* c, int32_t layer, int32_t B,
                           const int32_t* d_new_offsets, const int32_t* d_start_pos,
                           const int32_t* d_page_table, int32_t max_pages, const void* k_new,
                           const void* v_new, int64_t row_stride, int32_t n_new_total,
                           hipStream_t stream) {
  if (!c || !c->k_pool) return fail(HSTU_ERR_INVALID, "kv_page_append: cache without pools");
  if (layer < 0 || layer >= c->num_layers || B < 0 || max_pages <= 0 || n_new_total < 0)
    return fail(HSTU_ERR_INVALID, "kv_page_append: bad layer/B/max_pages/n_new_total");
  if (row_stride < static_cast<int64_t>(c->num_heads) * c->head_dim)
    return fail(HSTU_ERR_INVALID, "kv_page_append: row_stride smaller than a row");
  if (n_new_total == 0) return ok();
  if (!d_new_offsets || !d_start_pos || !d_page_table || !k_new || !v_new)
    return fail(HSTU_ERR_INVALID, "kv_page_append: null device pointer");
  if (row_stride % 8 != 0 || reinterpret_cast<uintptr_t>(k_new) % 16 ||
      reinterpret_cast<uintptr_t>(v_new) % 16)
    return fail(HSTU_ERR_INVALID, "kv_page_append: rows must be 16-byte aligned");
  return check_hip(timed(TK_APPEND, stream, [&] { return launch_append(c->dtype, nullptr, B, d_new_offsets, d_start_pos, d_page_table,
                                 max_pages, k_new, v_new, row_stride, n_new_total, c->k_pool,
                                 c->v_pool, layer, c->num_pages, c->num_heads, c->head_dim,
                                 c->page_size, stream); }),
                   "kv_page_append");
}

hstu_status kv_page_gather(const hstu_kv_cache* c, int32_t layer, int32_t B,
                           const int32_t* d_page_table, int32_t max_pages, const int32_t* d_kv_len,
                           const int32_t* d_out_offsets, int32_t n_out_total, void* k_out,
                           void* v_out, hipStream_t stream) {
  if (!c || !c->k_pool) return fail(HSTU_ERR_INVALID, "kv_page_gather: cache without pools");
  if (layer < 0 || layer >= c->num_layers || B < 0 || max_pages <= 0 || n_out_total < 0)
    return fail(HSTU_ERR_INVALID, "kv_page_gather: bad layer/B/max_pages/n_out_total");
  if (n_out_total == 0) return ok();
  if (!d_page_table || !d_kv_len || !d_out_offsets || !k_out || !v_out)
    return fail(HSTU_ERR_INVALID, "kv_page_gather: null device pointer");
  return check_hip(timed(TK_GATHER, stream, [&] { return launch_gather(c->dtype, B, d_page_table, max_pages, d_kv_len, d_out_offsets,
                                 n_out_total, k_out, v_out, c->k_pool, c->v_pool, layer,
                                 c->num_pages, c->num_heads, c->head_dim, c->page_size, stream); }),
                   "kv_page_gather");
}

// ---------------------------------------------------------------------------
// attention and layer
// ---------------------------------------------------------------------------

static hstu_status check_plan(const hstu_plan* p, const char* who) {
  if (!p) return fail(HSTU_ERR_INVALID, std::string(who) + ": null plan");
  if (!p->d_meta) return fail(HSTU_ERR_INVALID, std::string(who) + ": plan not uploaded");
  return HSTU_OK;
}

static hstu_status check_dtype_shape(int dtype, int dh, const char* who) {
  if (dtype != HSTU_F32 && dtype != HSTU_BF16)
    return fail(HSTU_ERR_INVALID, std::string(who) + ": unknown dtype");
  if (dtype == HSTU_BF16 && dh != 128)
    return fail(HSTU_ERR_UNSUPPORTED, std::string(who) + ": bf16 needs head_dim 128");
  return HSTU_OK;
}

static hstu_status fill_keys(AttnLaunch& L, const hstu_plan* p, int dtype, const void* k,
                             const void* v, int64_t kv_stride, const hstu_kv_cache* cache,
                             int32_t layer, const int32_t* d_pt, const char* who) {
  const int H = p->desc.num_heads, dh = p->desc.head_dim;
  if (p->desc.page_size > 0) {
    if (!cache || !cache->k_pool || !d_pt)
      return fail(HSTU_ERR_INVALID, std::string(who) + ": paged plan needs a cache and page table");
    if (cache->page_size != p->desc.page_size || cache->num_heads != H ||
        cache->head_dim != dh || cache->dtype != dtype)
      return fail(HSTU_ERR_INVALID, std::string(who) + ": cache geometry differs from the plan");
    if (layer < 0 || layer >= cache->num_layers)
      return fail(HSTU_ERR_INVALID, std::string(who) + ": bad layer");
    const int P = cache->page_size;
    if (dtype == HSTU_BF16 && (P < 16 || (P & (P - 1)) != 0))
      return fail(HSTU_ERR_UNSUPPORTED, std::string(who) + ": bf16 pages must hold a power of two >= 16 tokens");
    L.k_pool = cache->k_pool;
    L.v_pool = cache->v_pool;
    L.pool_layer_offset =
        static_cast<int64_t>(layer) * cache->num_pages * H * cache->page_size * dh;
    L.num_pages = cache->num_pages;
    L.page_table = d_pt;
  } else {
    if (!k || !v) return fail(HSTU_ERR_INVALID, std::string(who) + ": contiguous plan needs k and v");
    if (kv_stride < static_cast<int64_t>(H) * dh || kv_stride % 8)
      return fail(HSTU_ERR_INVALID, std::string(who) + ": bad kv_row_stride");
    L.k = k;
    L.v = v;
    L.kv_stride = kv_stride;
  }
  return HSTU_OK;
}

// The attention launch of a plan: one grid, or in split timing mode, when
// the plan mixes users with and without a cached prefix, its two orders as
// two grids timed apart (the same items, so the same results).
static hipError_t run_attention(const hstu_plan* p, const AttnLaunch& L0, hipStream_t s) {
  AttnLaunch L = L0;
  if (L.dtype == HSTU_BF16) L.stamps = attn_stamps_for(p->dev.n_items);
  if (timing_mode() == 2 && !p->items_split.empty()) {
    AttnLaunch A = L;
    A.stamps = nullptr;
    A.plan.items = p->d_items_split;
    A.plan.n_items = p->n_split_cached;
    hipError_t e = timed(TK_ATTN_CACHED, s, [&] { return launch_attention(A, s); });
    if (e != hipSuccess) return e;
    A.plan.items = p->d_items_split + p->n_split_cached;
    A.plan.n_items = static_cast<int32_t>(p->items_split.size()) - p->n_split_cached;
    return timed(TK_ATTN_PREFILL, s, [&] { return launch_attention(A, s); });
  }
  return timed(TK_ATTENTION, s, [&] { return launch_attention(L, s); });
}

}  // extern "C"

namespace hstu {
hstu_status attn_fwd_into(const hstu_attn_args* a, void* partials, size_t partial_bytes, hipStream_t stream,
                          const char* who) {
  if (!a) return fail(HSTU_ERR_INVALID, std::string(who) + ": null args");
  hstu_status st = check_plan(a->plan, who);
  if (st != HSTU_OK) return st;
  const hstu_plan* p = a->plan;
  const int H = p->desc.num_heads, dh = p->desc.head_dim;
  if ((st = check_dtype_shape(a->dtype, dh, who)) != HSTU_OK) return st;
  if (p->n_new == 0) return ok();
  if (!a->q || !a->out || !a->rab || a->num_buckets <= 0)
    return fail(HSTU_ERR_INVALID, std::string(who) + ": null q/out/rab or no buckets");
  if (a->num_buckets > 256) return fail(HSTU_ERR_UNSUPPORTED, std::string(who) + ": more than 256 buckets");
  if (a->q_row_stride < static_cast<int64_t>(H) * dh || a->q_row_stride % 8)
    return fail(HSTU_ERR_INVALID, std::string(who) + ": bad q_row_stride");
  hstu_plan_info info{};
  hstu_plan_get_info(p, &info);
  if (!partials || partial_bytes < info.attn_workspace_bytes)
    return fail(HSTU_ERR_INVALID, std::string(who) + ": workspace too small");
  AttnLaunch L{};
  L.dtype = a->dtype;
  L.plan = p->dev;
  L.q = a->q;
  L.q_stride = a->q_row_stride;
  L.rab = a->rab;
  L.num_buckets = a->num_buckets;
  L.partials = partials;
  if ((st = fill_keys(L, p, a->dtype, a->k, a->v, a->kv_row_stride, a->cache, a->layer,
                      a->d_page_table, who)) != HSTU_OK)
    return st;
  if ((st = check_hip(run_attention(p, L, stream), "attention")) != HSTU_OK) return fail(st, std::string(who) + ": " + g_last_error);
  if ((st = check_hip(timed(TK_REDUCE, stream, [&] { return launch_reduce_gate(a->dtype, p->dev, L.partials, partial_scale(a->dtype), nullptr, 0, 0.f, a->out,
                                      nullptr, stream); }),
                      "reduce")) != HSTU_OK)
    return fail(st, std::string(who) + ": " + g_last_error);
  return ok();
}
}  // namespace hstu

extern "C" {

hstu_status hstu_attn_stamps(void* d_stamps, int64_t capacity) {
  if (capacity < 0 || (capacity > 0 && !d_stamps)) return fail(HSTU_ERR_INVALID, "hstu_attn_stamps: bad buffer");
  if (reinterpret_cast<uintptr_t>(d_stamps) % 16) return fail(HSTU_ERR_INVALID, "hstu_attn_stamps: 16-byte alignment");
  int dev = -1;
  if (capacity > 0) {
    hstu_status st = check_hip(hipGetDevice(&dev), "hstu_attn_stamps");
    if (st != HSTU_OK) return st;
  }
  std::lock_guard<std::mutex> lk(g_stamps_mu);
  g_stamps = capacity > 0 ? static_cast<AttnStamp*>(d_stamps) : nullptr;
  g_stamps_cap = capacity;
  g_stamps_dev = dev;
  return ok();
}

hstu_status hstu_attn_fwd(const hstu_attn_args* a, hipStream_t stream) {
  return attn_fwd_into(a, a ? a->workspace : nullptr, a ? a->workspace_bytes : 0, stream, "hstu_attn_fwd");
}

namespace {
struct LayerWs {
  size_t xhat, colsum, slots, uvqk, partials, g, total;
};
// bf16 keeps only the row statistics of x (8 bytes a row) and the column sums
// of W1 where fp32 keeps the normalised copy
LayerWs layer_ws(const hstu_plan* p, int dtype, int d_model) {
  const size_t n = static_cast<size_t>(p->n_new), inner = p->desc.num_heads * p->desc.head_dim;
  LayerWs w{};
  size_t off = 0;
  w.xhat = off;
  // bf16: row statistics [n] (one slot a row), the f1 column sums [4 inner]
  // fp32 and the rows' pool slots [n] int64
  w.colsum = align256(off + n * sizeof(RowStat) + 1);
  w.slots = align256(w.colsum + 4 * inner * sizeof(float) + 1);
  off = dtype == HSTU_BF16 ? align256(w.slots + n * sizeof(int64_t) + 1)
                           : align256(off + n * d_model * esize(dtype) + 1);
  w.uvqk = off;
  off = align256(off + n * 4 * inner * esize(dtype) + 1);
  w.partials = off;
  off = align256(off + static_cast<size_t>(p->n_slots) * kBlockQ * p->desc.head_dim * 4 + 1);
  w.g = off;
  off = align256(off + n * inner * esize(dtype) + 1);
  w.total = off;
  return w;
}
}  // namespace

hstu_status hstu_layer_workspace_size(const hstu_layer_args* a, size_t* bytes) {
  if (!a || !bytes || !a->plan) return fail(HSTU_ERR_INVALID, "hstu_layer_workspace_size: null");
  *bytes = layer_ws(a->plan, a->dtype, a->d_model).total;
  return ok();
}

hstu_status hstu_layer_forward(const hstu_layer_args* a, hipStream_t stream) {
  if (!a) return fail(HSTU_ERR_INVALID, "hstu_layer_forward: null args");
  hstu_status st = check_plan(a->plan, "hstu_layer_forward");
  if (st != HSTU_OK) return st;
  const hstu_plan* p = a->plan;
  const int H = p->desc.num_heads, dh = p->desc.head_dim, inner = H * dh, d = a->d_model;
  if ((st = check_dtype_shape(a->dtype, dh, "hstu_layer_forward")) != HSTU_OK) return st;
  if (d <= 0 || (a->dtype == HSTU_BF16 && d % 128 != 0) || (a->dtype == HSTU_F32 && d % 4 != 0))
    return fail(HSTU_ERR_UNSUPPORTED,
                "hstu_layer_forward: d_model must be a multiple of 128 (bf16) or 4 (fp32)");
  if (!(a->eps >= 0.f)) return fail(HSTU_ERR_INVALID, "hstu_layer_forward: eps must be >= 0");
  if (a->s_out && a->dtype != HSTU_BF16)
    return fail(HSTU_ERR_UNSUPPORTED, "hstu_layer_forward: the s_out tap is bf16 only");
  if ((a->x_stats || a->y_stats) && (a->dtype != HSTU_BF16 || d > 128 * kMaxStatSlots))
    return fail(HSTU_ERR_UNSUPPORTED, "hstu_layer_forward: x_stats / y_stats need bf16 and d_model <= 512");
  if (a->row_slots && a->dtype != HSTU_BF16)
    return fail(HSTU_ERR_UNSUPPORTED, "hstu_layer_forward: row_slots is bf16 only");
  if (a->x_stats && p->desc.page_size > 0 && !a->row_slots)
    return fail(HSTU_ERR_INVALID, "hstu_layer_forward: x_stats on a paged plan needs row_slots");
  if (p->n_new == 0) return ok();
  if (!a->x || !a->y || !a->w1 || !a->w2 || !a->rab || a->num_buckets <= 0)
    return fail(HSTU_ERR_INVALID, "hstu_layer_forward: null x/y/w1/w2/rab or no buckets");
  if (a->num_buckets > 256) return fail(HSTU_ERR_UNSUPPORTED, "hstu_layer_forward: more than 256 buckets");
  const size_t xbytes = static_cast<size_t>(p->n_new) * d * esize(a->dtype);
  {
    auto xb = reinterpret_cast<uintptr_t>(a->x), yb = reinterpret_cast<uintptr_t>(a->y);
    if (xb < yb + xbytes && yb < xb + xbytes)
      return fail(HSTU_ERR_INVALID, "hstu_layer_forward: y overlaps x");
  }
  if (p->desc.page_size == 0) {
    for (int32_t c : p->cached_len)
      if (c != 0)
        return fail(HSTU_ERR_INVALID, "hstu_layer_forward: contiguous plan with cached positions");
  }
  LayerWs w = layer_ws(p, a->dtype, d);
  if (!a->workspace || a->workspace_bytes < w.total)
    return fail(HSTU_ERR_INVALID, "hstu_layer_forward: workspace too small");
  if (reinterpret_cast<uintptr_t>(a->workspace) % 256)
    return fail(HSTU_ERR_INVALID, "hstu_layer_forward: workspace must be 256-byte aligned");
  auto* ws = static_cast<unsigned char*>(a->workspace);
  void* xhat = ws + w.xhat;
  auto* uvqk = static_cast<unsigned char*>(a->uvqk_out ? a->uvqk_out : ws + w.uvqk);
  void* partials = ws + w.partials;
  void* g = a->g_out ? a->g_out : ws + w.g;
  const size_t es = esize(a->dtype);
  const int32_t M = p->n_new;

  const void* v_new = uvqk + static_cast<size_t>(inner) * es;
  const void* q_new = uvqk + static_cast<size_t>(2 * inner) * es;
  const void* k_new = uvqk + static_cast<size_t>(3 * inner) * es;
  AttnLaunch L{};
  L.dtype = a->dtype;
  L.plan = p->dev;
  L.q = q_new;
  L.q_stride = 4 * inner;
  L.rab = a->rab;
  L.num_buckets = a->num_buckets;
  L.partials = partials;
  const bool paged = p->desc.page_size > 0;
  if (paged) {
    if ((st = fill_keys(L, p, a->dtype, nullptr, nullptr, 0, a->cache, a->layer, a->d_page_table,
                        "hstu_layer_forward")) != HSTU_OK)
      return st;
  } else {
    if ((st = fill_keys(L, p, a->dtype, k_new, v_new, 4 * inner, nullptr, 0, nullptr,
                        "hstu_layer_forward")) != HSTU_OK)
      return st;
  }
  const hstu_kv_cache* c = a->cache;
  if (a->dtype == HSTU_BF16) {
    // row statistics (unless the previous layer's f2 left them) and W1's
    // column sums (unless precomputed), then f1 with the pre-norm, SiLU and
    // the K/V append fused
    auto* row_stats = static_cast<RowStat*>(xhat);
    float* colsum = reinterpret_cast<float*>(ws + w.colsum);
    F1Args f{};
    f.uvqk = uvqk;
    f.inner = inner;
    f.kv_to_uvqk = a->uvqk_out != nullptr;
    f.s_out = a->s_out;
    f.dh = dh;
    f.eps = a->eps;
    // the rows' pool slots: looked up with the statistics, or the caller's
    // from an earlier layer of the request
    RowSlots sl{};
    int64_t* row_slots = a->row_slots ? a->row_slots : reinterpret_cast<int64_t*>(ws + w.slots);
    if (paged) {
      f.k_pool = c->k_pool;
      f.v_pool = c->v_pool;
      f.pool_layer_offset = L.pool_layer_offset;
      f.page_size = c->page_size;
      f.row_slots = row_slots;
      if (!a->x_stats) {
        sl.out = row_slots;
        sl.row_pos = p->dev.row_pos;
        sl.page_table = a->d_page_table;
        sl.max_pages = p->desc.max_pages;
        sl.num_pages = c->num_pages;
        sl.H = H;
        sl.dh = dh;
        sl.page_size = c->page_size;
      }
    }
    const int32_t stat_rows = a->x_stats ? 0 : M;
    const int32_t cs_rows = a->w1_colsum ? 0 : 4 * inner;
    const RowStat* x_stats = a->x_stats ? reinterpret_cast<const RowStat*>(a->x_stats) : row_stats;
    const int32_t slots = a->x_stats ? d / 128 : 1;
    if (a->w1_colsum) colsum = const_cast<float*>(a->w1_colsum);
    if ((stat_rows || cs_rows) &&
        (st = check_hip(timed(TK_LAYER_NORM, stream, [&] { return launch_row_stats(a->x, row_stats, stat_rows, d, a->w1, colsum, cs_rows, sl, stream); }),
                        "hstu_layer_forward: row statistics")) != HSTU_OK)
      return st;
    if ((st = check_hip(timed(TK_F1, stream, [&] { return launch_f1_bf16(a->x, x_stats, slots, colsum, a->w1, f, M, 4 * inner, d, stream); }),
                        "hstu_layer_forward: f1")) != HSTU_OK)
      return st;
  } else {
    if ((st = check_hip(timed(TK_LAYER_NORM, stream, [&] { return launch_layer_norm(a->dtype, a->x, xhat, M, d, a->eps, stream); }),
                        "hstu_layer_forward: pre-norm")) != HSTU_OK)
      return st;
    if ((st = check_hip(timed(TK_F1, stream, [&] { return launch_gemm(a->dtype, 0, xhat, a->w1, uvqk, nullptr, M, 4 * inner, d, stream); }),
                        "hstu_layer_forward: f1")) != HSTU_OK)
      return st;
    if (paged &&
        (st = check_hip(timed(TK_APPEND, stream, [&] { return launch_append(a->dtype, &p->dev, p->desc.B, p->dev.new_offsets,
                                      p->dev.start_pos, a->d_page_table, p->desc.max_pages, k_new,
                                      v_new, 4 * inner, M, c->k_pool, c->v_pool, a->layer,
                                      c->num_pages, H, dh, c->page_size, stream); }),
                        "hstu_layer_forward: append")) != HSTU_OK)
      return st;
  }
  if ((st = check_hip(run_attention(p, L, stream), "hstu_layer_forward: attention")) != HSTU_OK)
    return st;
  if ((st = check_hip(timed(TK_REDUCE, stream, [&] { return launch_reduce_gate(a->dtype, p->dev, partials, partial_scale(a->dtype), uvqk, 4 * inner, a->eps,
                                         a->o_out, g, stream); }),
                      "hstu_layer_forward: LayerNorm gate")) != HSTU_OK)
    return st;
  return check_hip(timed(TK_F2, stream, [&] { return launch_gemm(a->dtype, 1, g, a->w2, a->y, a->x, M, d, inner, stream,
                                                                reinterpret_cast<RowStat*>(a->y_stats)); }),
                   "hstu_layer_forward: f2");
}

hstu_status hstu_stack_forward(const hstu_layer_args* layers, int32_t n, hipStream_t stream) {
  if (n < 0 || (n > 0 && !layers)) return fail(HSTU_ERR_INVALID, "hstu_stack_forward: bad layer list");
  for (int32_t i = 0; i < n; ++i) {
    hstu_status st = hstu_layer_forward(&layers[i], stream);
    if (st != HSTU_OK) return fail(st, "hstu_stack_forward: layer " + std::to_string(i) + ": " + g_last_error);
  }
  return ok();
}

hstu_status hstu_w1_colsum(const void* w1, int32_t rows, int32_t d_model, float* out, hipStream_t stream) {
  if (!w1 || !out || rows <= 0 || d_model <= 0 || d_model % 8 || d_model > 2048)
    return fail(HSTU_ERR_INVALID, "hstu_w1_colsum: bad arguments");
  // no statistics rows: only the column-sum blocks run
  return check_hip(launch_row_stats(nullptr, nullptr, 0, d_model, w1, out, rows, RowSlots{}, stream),
                   "hstu_w1_colsum");
}

// ---------------------------------------------------------------------------
// backward of one layer
// ---------------------------------------------------------------------------

namespace {
struct BwdWs {
  size_t dg, dout, g, da, dxh, xhat, zeros, part, drab_part, kv_items, q_items, total;
  int32_t n_kv, n_q, splits1, splits2;
};
constexpr int kBwdKeys = kBwdKeyBlock;
constexpr int kWgradTile = 128;

int32_t wgrad_splits(int32_t M, int32_t N1, int32_t N2) {
  const int32_t tiles = (N1 / kWgradTile) * (N2 / kWgradTile);
  int32_t s = (512 + tiles - 1) / tiles;
  const int32_t max_s = std::max(1, (M + 63) / 64);
  return std::max(1, std::min(s, max_s));
}

BwdWs bwd_ws(const hstu_plan* p, int32_t d) {
  const size_t n = static_cast<size_t>(p->n_new), inner = p->desc.num_heads * p->desc.head_dim;
  BwdWs w{};
  w.n_kv = 0;
  for (size_t u = 0; u < p->users.size(); ++u)
    w.n_kv += (p->users[u].kv_len + kBwdKeys - 1) / kBwdKeys * p->desc.num_heads;
  w.n_q = static_cast<int32_t>(p->qblocks.size()) * p->desc.num_heads;
  const int32_t M = p->n_new, W = static_cast<int32_t>(4 * inner);
  w.splits1 = wgrad_splits(M, W, d);
  w.splits2 = wgrad_splits(M, d, static_cast<int32_t>(inner));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes + 1);
    return at;
  };
  w.dg = take(n * inner * 2);
  w.dout = take(n * inner * 2);
  w.g = take(n * inner * 2);
  w.da = take(n * 4 * inner * 2);
  w.dxh = take(n * d * 2);
  w.xhat = take(n * d * 2);
  w.zeros = take(256 * 2);
  w.part = take(std::max(static_cast<size_t>(w.splits1) * W * d, static_cast<size_t>(w.splits2) * d * inner) * 4);
  w.drab_part = take(static_cast<size_t>(w.n_kv) * 256 * 4);
  w.kv_items = take(static_cast<size_t>(w.n_kv) * sizeof(BwdKVItem));
  w.q_items = take(static_cast<size_t>(w.n_q) * sizeof(BwdQItem));
  w.total = off;
  return w;
}

hstu_status bwd_check(const hstu_layer_bwd_args* a, const char* who) {
  if (!a) return fail(HSTU_ERR_INVALID, std::string(who) + ": null args");
  hstu_status st = check_plan(a->plan, who);
  if (st != HSTU_OK) return st;
  const hstu_plan* p = a->plan;
  if (a->dtype != HSTU_BF16) return fail(HSTU_ERR_UNSUPPORTED, std::string(who) + ": bf16 only");
  if (p->desc.head_dim != 128 || p->desc.num_heads * p->desc.head_dim > 512)
    return fail(HSTU_ERR_UNSUPPORTED, std::string(who) + ": head_dim 128 and H*head_dim <= 512 only");
  if (a->d_model <= 0 || a->d_model % 128 || a->d_model > 2048)
    return fail(HSTU_ERR_UNSUPPORTED, std::string(who) + ": d_model must be a multiple of 128, <= 2048");
  if (p->desc.page_size != 0) return fail(HSTU_ERR_UNSUPPORTED, std::string(who) + ": paged plans are not supported");
  for (int32_t c : p->cached_len)
    if (c != 0) return fail(HSTU_ERR_UNSUPPORTED, std::string(who) + ": cached positions are not supported");
  if (a->num_buckets <= 0 || a->num_buckets > 256)
    return fail(HSTU_ERR_INVALID, std::string(who) + ": num_buckets must be in [1, 256]");
  if (!(a->eps >= 0.f)) return fail(HSTU_ERR_INVALID, std::string(who) + ": eps must be >= 0");
  return HSTU_OK;
}
}  // namespace

hstu_status hstu_layer_backward_workspace_size(const hstu_layer_bwd_args* a, size_t* bytes) {
  if (!bytes) return fail(HSTU_ERR_INVALID, "hstu_layer_backward_workspace_size: null output");
  hstu_status st = bwd_check(a, "hstu_layer_backward_workspace_size");
  if (st != HSTU_OK) return st;
  *bytes = bwd_ws(a->plan, a->d_model).total;
  return ok();
}

hstu_status hstu_layer_backward(const hstu_layer_bwd_args* a, hipStream_t stream) {
  hstu_status st = bwd_check(a, "hstu_layer_backward");
  if (st != HSTU_OK) return st;
  const hstu_plan* p = a->plan;
  const int32_t M = p->n_new, d = a->d_model, H = p->desc.num_heads, inner = H * p->desc.head_dim, W = 4 * inner;
  if (!a->x || !a->w1t || !a->w2t || !a->rab || !a->uvqk || !a->s || !a->o || !a->dy || !a->dx || !a->dw1 ||
      !a->dw2 || !a->drab)
    return fail(HSTU_ERR_INVALID, "hstu_layer_backward: null buffer");
  BwdWs w = bwd_ws(p, d);
  if (!a->workspace || a->workspace_bytes < w.total)
    return fail(HSTU_ERR_INVALID, "hstu_layer_backward: workspace too small");
  if (reinterpret_cast<uintptr_t>(a->workspace) % 256)
    return fail(HSTU_ERR_INVALID, "hstu_layer_backward: workspace must be 256-byte aligned");
  auto* ws = static_cast<unsigned char*>(a->workspace);
  void* dg = ws + w.dg;
  void* dout = ws + w.dout;
  void* g = ws + w.g;
  void* da = ws + w.da;
  void* dxh = ws + w.dxh;
  void* xhat = ws + w.xhat;
  void* zeros = ws + w.zeros;
  float* part = reinterpret_cast<float*>(ws + w.part);
  float* drab_part = reinterpret_cast<float*>(ws + w.drab_part);

  // work lists: key blocks and query blocks of every (user, head), the
  // longest first (a key block's work grows with the queries after it)
  std::vector<BwdKVItem> kv;
  kv.reserve(static_cast<size_t>(w.n_kv));
  for (size_t u = 0; u < p->users.size(); ++u)
    for (int32_t k0 = 0; k0 < p->users[u].kv_len; k0 += kBwdKeys)
      for (int32_t h = 0; h < H; ++h) kv.push_back(BwdKVItem{static_cast<int32_t>(u), h, k0, 0});
  std::stable_sort(kv.begin(), kv.end(), [&](const BwdKVItem& x, const BwdKVItem& y) {
    return p->users[x.user].kv_len - x.k0 > p->users[y.user].kv_len - y.k0;
  });
  std::vector<BwdQItem> qi;
  qi.reserve(static_cast<size_t>(w.n_q));
  for (size_t q = 0; q < p->qblocks.size(); ++q)
    for (int32_t h = 0; h < H; ++h) qi.push_back(BwdQItem{static_cast<int32_t>(q), h});
  std::stable_sort(qi.begin(), qi.end(), [&](const BwdQItem& x, const BwdQItem& y) {
    return p->qblocks[x.qblock].pos0 + p->qblocks[x.qblock].count >
           p->qblocks[y.qblock].pos0 + p->qblocks[y.qblock].count;
  });
  if (!kv.empty() &&
      (st = staged_upload(ws + w.kv_items, kv.data(), kv.size() * sizeof(BwdKVItem), stream)) != HSTU_OK)
    return st;
  if (!qi.empty() &&
      (st = staged_upload(ws + w.q_items, qi.data(), qi.size() * sizeof(BwdQItem), stream)) != HSTU_OK)
    return st;

  const int64_t W64 = W;
  if ((st = check_hip(launch_fill_zero(zeros, 256, stream), "hstu_layer_backward: zeros")) != HSTU_OK) return st;
  if (M > 0) {
    if ((st = check_hip(timed(TK_BWD_GEMM, stream, [&] { return launch_gemm(HSTU_BF16, 3, a->dy, a->w2t, dg, nullptr, M, inner, d, stream); }),
                        "hstu_layer_backward: dg")) != HSTU_OK)
      return st;
    if ((st = check_hip(timed(TK_BWD_ROWS, stream, [&] { return launch_gate_bwd(a->o, a->uvqk, W64, dg, M, inner, a->eps, da, dout, g, stream); }),
                        "hstu_layer_backward: gate")) != HSTU_OK)
      return st;
    BwdLaunch b{};
    b.plan = p->dev;
    b.a = static_cast<const uint16_t*>(a->uvqk);
    b.dO = static_cast<const uint16_t*>(dout);
    b.da = static_cast<uint16_t*>(da);
    b.rab = a->rab;
    b.num_buckets = a->num_buckets;
    b.drab_partial = drab_part;
    b.kv_items = reinterpret_cast<const BwdKVItem*>(ws + w.kv_items);
    b.n_kv_items = static_cast<int32_t>(kv.size());
    b.q_items = reinterpret_cast<const BwdQItem*>(ws + w.q_items);
    b.n_q_items = static_cast<int32_t>(qi.size());
    if ((st = check_hip(timed(TK_BWD_ATTENTION, stream, [&] {
                          hipError_t e = launch_attn_bwd(b, stream);
                          return e != hipSuccess ? e : launch_drab_sum(drab_part, b.n_kv_items, a->num_buckets, a->drab, stream);
                        }),
                        "hstu_layer_backward: attention")) != HSTU_OK)
      return st;
    if ((st = check_hip(timed(TK_BWD_ROWS, stream, [&] { return launch_silu_grad(da, a->s, static_cast<int64_t>(M) * W, stream); }),
                        "hstu_layer_backward: SiLU'")) != HSTU_OK)
      return st;
    if ((st = check_hip(timed(TK_BWD_GEMM, stream, [&] { return launch_gemm(HSTU_BF16, 3, da, a->w1t, dxh, nullptr, M, d, W, stream); }),
                        "hstu_layer_backward: dx^")) != HSTU_OK)
      return st;
    if ((st = check_hip(timed(TK_BWD_ROWS, stream, [&] { return launch_ln_bwd(a->x, dxh, a->dy, M, d, a->eps, a->dx, xhat, stream); }),
                        "hstu_layer_backward: pre-norm")) != HSTU_OK)
      return st;
  } else {
    if ((st = check_hip(launch_drab_sum(drab_part, 0, a->num_buckets, a->drab, stream), "hstu_layer_backward: drab")) != HSTU_OK)
      return st;
  }
  if ((st = check_hip(timed(TK_BWD_GEMM, stream, [&] { return launch_wgrad(a->dy, d, g, inner, M, d, inner, w.splits2, zeros, part, a->dw2, stream); }),
                      "hstu_layer_backward: dW2")) != HSTU_OK)
    return st;
  return check_hip(timed(TK_BWD_GEMM, stream, [&] { return launch_wgrad(da, W64, xhat, d, M, W, d, w.splits1, zeros, part, a->dw1, stream); }),
                   "hstu_layer_backward: dW1");
}

// ---------------------------------------------------------------------------
// multitask ranking head
// ---------------------------------------------------------------------------

namespace {
hstu_status head_check(const hstu_head_args* a, size_t* need) {
  if (!a) return fail(HSTU_ERR_INVALID, "hstu_head: null arguments");
  if (a->dtype != HSTU_BF16) return fail(HSTU_ERR_UNSUPPORTED, "hstu_head: only bf16 is supported");
  if (a->d_model <= 0 || a->d_model % 64 != 0 || a->num_tasks <= 0 || a->hidden <= 0 ||
      a->hidden % kHeadTile != 0 || a->n_rows < 0)
    return fail(HSTU_ERR_INVALID, "hstu_head: d_model must be a multiple of 64, hidden of 128");
  if (static_cast<int64_t>(a->num_tasks) * a->hidden > (1 << 30))
    return fail(HSTU_ERR_INVALID, "hstu_head: too many hidden units");
  *need = align256(static_cast<size_t>(a->n_rows) * a->num_tasks * (a->hidden / kHeadTile) * sizeof(float));
  return ok();
}
}  // namespace

hstu_status hstu_head_workspace_size(const hstu_head_args* a, size_t* bytes) {
  if (!bytes) return fail(HSTU_ERR_INVALID, "hstu_head_workspace_size: null output");
  return head_check(a, bytes);
}

hstu_status hstu_head_forward(const hstu_head_args* a, hipStream_t stream) {
  size_t need = 0;
  hstu_status st = head_check(a, &need);
  if (st != HSTU_OK) return st;
  if (a->n_rows == 0) return ok();
  if (a->y_rows <= 0 || !a->y || !a->d_rows || !a->w_hidden || !a->b_hidden || !a->w_out || !a->b_out ||
      !a->logits)
    return fail(HSTU_ERR_INVALID, "hstu_head_forward: null buffer or no rows in y");
  if (!a->workspace || a->workspace_bytes < need)
    return fail(HSTU_ERR_INVALID, "hstu_head_forward: workspace too small");
  HeadArgs h{};
  h.y = a->y;
  h.y_rows = a->y_rows;
  h.d = a->d_model;
  h.rows = a->d_rows;
  h.n_rows = a->n_rows;
  h.tasks = a->num_tasks;
  h.hidden = a->hidden;
  h.w_hidden = a->w_hidden;
  h.b_hidden = a->b_hidden;
  h.w_out = a->w_out;
  h.b_out = a->b_out;
  h.logits = a->logits;
  h.partial = static_cast<float*>(a->workspace);
  return check_hip(timed(TK_HEAD, stream, [&] { return launch_head_bf16(h, stream); }), "hstu_head_forward");
}

}  // extern "C"

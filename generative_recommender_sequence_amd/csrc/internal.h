// Internal declarations of libhstu: error state, the request plan's device
// records, and the kernel launchers the ABI layer calls.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>
#include <deque>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/hstu.h"

namespace hstu {

// ---- error reporting ------------------------------------------------------
hstu_status fail(hstu_status st, const std::string& msg);
hstu_status ok();
hstu_status check_hip(hipError_t e, const char* what);
// asynchronous host-to-device copy through a pinned staging buffer
hstu_status staged_upload(void* dst, const void* src, size_t bytes, hipStream_t stream);

// ---- tiling constants shared by the plan and the attention kernels --------
constexpr int kBlockQ = 128;  // queries per attention work item (4 waves x 32)
constexpr int kTileK = 64;    // keys per staged K/V tile
constexpr int kMaxPos = 65535;
// Page-table entries one paged work item may stage in LDS: the pages from
// the one holding its first key tile to the one holding its last.  The plan
// cuts every piece whose span would exceed it (a piece can skip a masked gap
// between history and candidate tiles, so its span is not bounded by its
// tile count alone).
constexpr int kMaxItemPages = 2048;

// One attention work item: a block of up to kBlockQ queries of one user and
// head, over the key tiles [tile_begin, tile_end) of that user.  Its result
// (unnormalised sum over those keys) goes to partial slot `slot`.  It carries
// the fields of its q-block and user that the kernels read, so that one
// load brings everything.
struct WorkItem {
  int32_t user, head, qblock, tile_begin, tile_end, slot;
  int32_t row0, count, pos0;     // the q-block: first row, queries, first position
  int32_t kv_len, hist, kv_row0;  // the user: keys, history length, first key row (contiguous)
  int32_t pad[4];
};

// The partial slots of one (q-block, head): consecutive, in key order.
struct SlotRange {
  int32_t first, count;
};

// A block of up to kBlockQ consecutive new tokens of one user.
struct QBlock {
  int32_t user, row0, count, pos0;
};

// User and sequence position of a new-token row.
struct RowPos {
  int32_t user, pos;
};

// Per-user scalars the kernels read.
struct UserInfo {
  int32_t q_row0;     // first new-token row
  int32_t n_new;      // t_u
  int32_t start;      // c_u (position of the first new token)
  int32_t kv_len;     // L_u = c_u + t_u
  int32_t hist;       // L_u - T_u
  int32_t kv_row0;    // contiguous mode: first key row
  float inv_n;        // 1 / n_u
  float pad;
};

// Device view of an uploaded plan (all pointers into the caller's d_meta).
struct PlanDev {
  const WorkItem* items;
  const QBlock* qblocks;
  const SlotRange* qb_slots;  // [n_qblocks][H]
  const UserInfo* users;
  const RowPos* row_pos;      // [n_new]
  const int32_t* new_offsets; // [B+1]
  const int32_t* start_pos;   // [B]
  int32_t n_items, n_qblocks, n_new, B, H, dh, page_size, max_pages, max_len;
};

}  // namespace hstu

struct hstu_plan {
  hstu_batch_desc desc{};
  std::vector<int32_t> new_len, cached_len, n_targets;
  std::vector<float> norm_n;
  std::vector<hstu::WorkItem> items;
  // items again as two dispatch orders (users with a cached prefix, then the
  // rest), when the request has both kinds; empty otherwise
  std::vector<hstu::WorkItem> items_split;
  int32_t n_split_cached = 0;
  std::vector<hstu::QBlock> qblocks;
  std::vector<hstu::SlotRange> qb_slots;
  std::vector<hstu::UserInfo> users;
  std::vector<hstu::RowPos> row_pos;
  std::vector<int32_t> new_offsets, start_pos;
  int32_t n_slots = 0, n_new = 0, max_len = 0;
  int64_t pairs = 0;
  std::vector<unsigned char> host_blob;  // packed image of the device metadata
  size_t off_items = 0, off_items_split = 0, off_qblocks = 0, off_qb_slots = 0, off_users = 0, off_row_pos = 0,
         off_new_offsets = 0, off_start_pos = 0;
  void* d_meta = nullptr;  // set by hstu_plan_upload
  const hstu::WorkItem* d_items_split = nullptr;
  hstu::PlanDev dev{};
};

struct hstu_kv_cache {
  struct User {
    int32_t len = 0;
    int64_t tick = 0;
    std::vector<int32_t> pages;
  };
  int32_t num_layers = 0, num_heads = 0, head_dim = 0, page_size = 0, num_pages = 0, dtype = 0;
  void* k_pool = nullptr;
  void* v_pool = nullptr;
  int64_t tick = 0;
  std::deque<int32_t> free_q;
  std::unordered_map<int64_t, User> users;  // device-resident users
  // host tier (host_pages < 0: none attached)
  int32_t host_pages = -1;
  void* host_k = nullptr;  // device-visible addresses of the caller's pinned host pools
  void* host_v = nullptr;
  std::deque<int32_t> host_free_q;
  std::unordered_map<int64_t, User> host_users;
};

namespace hstu {

// ---- optional event timing of launches (hstu_timing_*) ---------------------
enum TimedKernel { TK_LAYER_NORM, TK_F1, TK_APPEND, TK_ATTENTION, TK_REDUCE, TK_F2, TK_GATHER, TK_HEAD,
                   TK_BWD_ATTENTION, TK_BWD_GEMM, TK_BWD_ROWS, TK_ATTN_CACHED, TK_ATTN_PREFILL, TK_COUNT };
// 0: off; 1: every launch timed; 2: as 1, and an attention over users of
// both regimes (with and without a cached prefix) runs as two timed grids
int timing_mode();
// Brackets one launch: records a start event now and an end event when the
// returned guard's end() is called (both on stream s), if timing is enabled.
struct TimedLaunch {
  TimedLaunch(TimedKernel k, hipStream_t s);
  void end();
  int kernel;
  hipStream_t stream;
  void* start_ev;
};

// ---- kernel launchers (kernels/*.hip) -------------------------------------
// All take device pointers and enqueue on `s`; they return the launch status.
hipError_t launch_append(int dtype, const PlanDev* plan_or_null, int32_t B,
                         const int32_t* d_new_offsets, const int32_t* d_start_pos,
                         const int32_t* d_page_table, int32_t max_pages, const void* k_new,
                         const void* v_new, int64_t row_stride, int32_t n_new_total, void* k_pool,
                         void* v_pool, int32_t layer, int32_t num_pages, int32_t H, int32_t dh,
                         int32_t page_size, hipStream_t s);
// Copies whole pages (all heads) of every layer, K and V, between two pools:
// pairs (host pinned, device-visible) [n_pairs] of (source page, destination
// page); each pool is [layers][pages][page_bytes].
struct PagePair {
  int32_t src, dst;
};
hipError_t launch_tier_copy(const PagePair* pairs, int32_t n_pairs, int32_t layers, const void* src_k,
                            const void* src_v, int64_t src_pages, void* dst_k, void* dst_v,
                            int64_t dst_pages, int64_t page_bytes, hipStream_t s);
// Copies `bytes` of src into a pinned staging slot and calls use(slot) with
// the slot's (device-visible) address; the slot is reused only after the work
// `use` enqueued on `stream` has finished.
hstu_status staged_host(const void* src, size_t bytes, hipStream_t stream,
                        hipError_t (*use)(const void* slot, void* ctx), void* ctx);
hipError_t launch_gather(int dtype, int32_t B, const int32_t* d_page_table, int32_t max_pages,
                         const int32_t* d_kv_len, const int32_t* d_out_offsets, int32_t n_out_total,
                         void* k_out, void* v_out, const void* k_pool, const void* v_pool,
                         int32_t layer, int32_t num_pages, int32_t H, int32_t dh, int32_t page_size,
                         hipStream_t s);

// One attention block's phase record (hstu_attn_stamps): realtime-clock
// stamps (100 MHz) at its start, after its set-up (work item, page-table
// slice, bias, first tiles staged), after its tile loop and at its end, and
// where it ran.
struct AttnStamp {
  uint64_t start, setup_done, loop_done, end;
  uint32_t hw_id;   // the HW_ID register (CU, shader engine, SIMD, wave slot)
  uint32_t xcc_id;  // the XCD the block ran on
  int32_t slot;     // the item's partial slot
  int32_t tiles;    // key tiles in the item's range
};

struct AttnLaunch {
  int dtype;
  PlanDev plan;
  const void* q;
  int64_t q_stride;
  // contiguous keys
  const void* k;
  const void* v;
  int64_t kv_stride;
  // paged keys
  const void* k_pool;
  const void* v_pool;
  int64_t pool_layer_offset;  // elements: layer * num_pages * H * page_size * dh
  int32_t num_pages;
  const int32_t* page_table;
  const float* rab;
  int32_t num_buckets;
  void* partials;  // fp32 [n_slots][kBlockQ][dh]
  AttnStamp* stamps;  // per-block phase records [n_items] (nullptr: none)
};
hipError_t launch_attention(const AttnLaunch& a, hipStream_t s);
// the phase-record buffer registered with hstu_attn_stamps (nullptr: none)
AttnStamp* attn_stamps_for(int32_t n_items);
// hstu_attn_fwd with its fp32 partial tiles in `partials` (partial_bytes
// long); errors name `who`
hstu_status attn_fwd_into(const hstu_attn_args* a, void* partials, size_t partial_bytes, hipStream_t stream,
                          const char* who);

// Sums each row's fp32 partial slots in key order, scales by o_scale / n_u;
// then writes o (fp32) and/or g = LayerNorm(o) * U (dtype).
hipError_t launch_reduce_gate(int dtype, const PlanDev& plan, const void* partials,
                              float o_scale, const void* u, int64_t u_stride, float eps,
                              float* o_out, void* g_out, hipStream_t s);
// The bf16 attention's partial sums carry a factor log2(e); this removes it.
constexpr float kBf16PartialScale = 0.693147180559945309f;
inline float partial_scale(int dtype) { return dtype == HSTU_BF16 ? kBf16PartialScale : 1.0f; }

// y = LayerNorm(x) rows (no affine) -> xhat (dtype)
hipError_t launch_layer_norm(int dtype, const void* x, void* xhat, int32_t rows, int32_t cols,
                             float eps, hipStream_t s);

// Statistics of a row of a bf16 activation, in slots: slot t holds the mean
// and the sum of squared deviations from it of the t-th of the row's equal
// column shares; the LayerNorm statistics combine them (the pairwise update
// of Chan, Golub and LeVeque).  f2 writes one slot per 128-column tile of its
// output (the next layer's input); the row-statistics kernel one slot per row.
struct RowStat {
  float mean, m2;
};
constexpr int kMaxStatSlots = 4;

// C[M][N] = epilogue(A[M][K] . Wt[N][K]^T); epilogue 0: SiLU, 1: + residual
// R[M][N], 3 (bf16 only): plain.  bf16 takes epilogues 1 and 3 (f1 goes
// through launch_f1_bf16); its epilogue 1 may also write the RowStat slots of
// C's rows, one per 128-column tile, to y_stats (nullptr: not kept).
hipError_t launch_gemm(int dtype, int epilogue, const void* A, const void* Bm, void* C,
                       const void* R, int32_t M, int32_t N, int32_t K, hipStream_t s,
                       RowStat* y_stats = nullptr);

// Where each new-token row's K/V go in one layer of the pools.
struct RowSlots {
  int64_t* out;               // [rows]: element offset of (page, head 0, slot), or -1 (nullptr: not computed)
  const RowPos* row_pos;      // [rows]
  const int32_t* page_table;  // [B][max_pages]
  int32_t max_pages, num_pages, H, dh, page_size;
};
// The statistics of each row of a bf16 [rows][cols] matrix as one RowStat
// slot (and the rows' pool slots if sl.out), and in the same launch the row
// sums of w1t (bf16 [w1t_rows][cols]) -> colsum
hipError_t launch_row_stats(const void* x, RowStat* stats, int32_t rows, int32_t cols, const void* w1t,
                            float* colsum, int32_t w1t_rows, const RowSlots& sl, hipStream_t s);

// Destinations of the bf16 f1 GEMM's output columns [U|V|Q|K].
struct F1Args {
  void* uvqk;             // [M][4 inner]: U and Q always; K and V if kv_to_uvqk or no pools
  int32_t inner;
  bool kv_to_uvqk;
  void* k_pool;           // paged K/V (nullptr: none), rows placed through the page table
  void* v_pool;
  int64_t pool_layer_offset;
  int32_t dh, page_size;
  void* s_out;            // optional [M][4 inner]: the pre-activation LayerNorm(x) . W1
  float eps;
  const int64_t* row_slots;   // [M] pool slot of each row (RowSlots::out), with k_pool
};
// [U|V|Q|K] = SiLU(LayerNorm(x) . W1) from raw x and its row statistics
// (RowStat [M][slots]), routed per F1Args
hipError_t launch_f1_bf16(const void* x, const RowStat* stats, int32_t slots, const float* colsum, const void* w1t,
                          const F1Args& f, int32_t M, int32_t N, int32_t K, hipStream_t s);

// Multitask ranking head on rows of y (bf16 [y_rows][d]): per task t and
// listed row, logit = b_out[t] + sum_j w_out[t][j] * ReLU(b_hidden[t][j] +
// y_row . w_hidden[t hidden + j]); w_hidden output-major [tasks*hidden][d].
constexpr int kHeadTile = 128;  // hidden columns per block (hidden % kHeadTile == 0)
struct HeadArgs {
  const void* y;
  int32_t y_rows, d;
  const int32_t* rows;  // [n_rows] (clamped to [0, y_rows))
  int32_t n_rows, tasks, hidden;
  const void* w_hidden;
  const float* b_hidden;  // [tasks*hidden]
  const float* w_out;     // [tasks*hidden]
  const float* b_out;     // [tasks]
  float* logits;          // [n_rows][tasks]
  float* partial;         // [n_rows][tasks*hidden/kHeadTile] scratch
};
hipError_t launch_head_bf16(const HeadArgs& h, hipStream_t s);

// ---- backward (training; contiguous keys, every position computed) ----
constexpr int kBwdKeyBlock = 64;  // keys per key-block item of the backward attention
struct BwdKVItem {
  int32_t user, head, k0, pad;  // kBwdKeyBlock keys from position k0
};
struct BwdQItem {
  int32_t qblock, head;
};
struct BwdLaunch {
  PlanDev plan;
  const uint16_t* a;      // [N][4 inner] post-SiLU [U|V|Q|K]
  const uint16_t* dO;     // [N][inner] gradient of o (o includes 1/n)
  uint16_t* da;           // [N][4 inner]: the attention writes the V, Q and K chunks
  const float* rab;
  int32_t num_buckets;
  float* drab_partial;    // [n_kv_items][num_buckets]
  const BwdKVItem* kv_items;
  int32_t n_kv_items;
  const BwdQItem* q_items;
  int32_t n_q_items;
};
hipError_t launch_attn_bwd(const BwdLaunch& b, hipStream_t s);
hipError_t launch_drab_sum(const float* part, int32_t items, int32_t nb, float* drab, hipStream_t s);
hipError_t launch_gate_bwd(const float* o, const void* a, int64_t a_stride, const void* dg, int32_t rows,
                           int32_t inner, float eps, void* du, void* dout, void* g, hipStream_t s);
hipError_t launch_ln_bwd(const void* x, const void* dxh, const void* dy, int32_t rows, int32_t d, float eps,
                         void* dx, void* xhat, hipStream_t s);
hipError_t launch_silu_grad(void* da, const void* s_pre, int64_t n, hipStream_t s);
hipError_t launch_fill_zero(void* p, int32_t n, hipStream_t s);
// out[i][j] = sum_m A[m][i] B[m][j] (fp32), split over m into `splits` chunks
// whose partials [splits][N1][N2] go to `part`; rows past M read `zeros`
hipError_t launch_wgrad(const void* A, int64_t lda, const void* B, int64_t ldb, int32_t M, int32_t N1, int32_t N2,
                        int32_t splits, const void* zeros, float* part, float* out, hipStream_t s);

// ---- achievable-ceiling kernels (kernels/ceiling.hip) ----
hipError_t launch_ceiling_mfma(int32_t blocks, int32_t iters, float* out, hipStream_t s);
hipError_t launch_ceiling_read(const void* src, int64_t bytes, void* out, hipStream_t s);
hipError_t launch_ceiling_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);

}  // namespace hstu

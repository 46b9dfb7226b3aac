// HSTU pointwise attention over jagged users with a cached prefix
// ("How Generative Recommenders Are Redefining RecSys at Scale", section
// HSTU: SiLU-based weighting instead of softmax normalisation, plus a relative
// attention bias; "Deploying an HSTU Generative Recommender with NVIDIA
// Dynamo-Triton", KV cache section: the attention reads the cached K/V
// directly).  Per head, for new-token query i of user u:
//     sum_{j in M(i)} SiLU(q_i . k_j + rab[b(i - j)]) * v_j
// M(i) = {j <= i} for history queries, {j < hist} u {i} for candidates.
// The 1/n_u scale is applied by the reduction that consumes the partials.
//
// Work item = (user, head, block of <= 128 queries, range of 64-key tiles),
// scheduled on the host.  Without a softmax there is no running max or
// rescale: each work item writes the plain sum over its keys into its own
// fp32 partial tile, and the reduction adds the tiles of a row in key order
// in fp32, so the result does not depend on scheduling.
//
// bf16 kernel (gfx950, 256 threads = 4 waves, 32 queries per wave):
//   S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 (keys are the M rows, queries
//   the N columns).  MFMA row i of a 32-key block reads key i with bits 2 and
//   3 swapped, so after SiLU each lane holds, for its own query, 8 consecutive
//   key weights per 16-key step: exactly one A operand of O += P . V.
//   K and V tiles are staged row-major in LDS (16-byte-chunk XOR swizzles);
//   the V operand is read with ds_read_b64_tr_b16, which hands each lane 4
//   consecutive keys of one column, so V is never transposed in registers.
//   The tiles are double-buffered and filled by direct global -> LDS copies
//   (no register staging): the next visible tile's copy is issued before the
//   current tile's MFMAs, and each tile costs one barrier.  The work item's
//   page-table slice is staged in LDS once (the first tile is addressed from
//   the table itself, so its copy goes out with the set-up loads).  The bias
//   of a tile comes from one scalar when a wave's distance range falls in a
//   single bucket, otherwise from a reversed per-tile table in LDS read with
//   immediate offsets, built only for tiles that need it.  Masking work is
//   only done on tiles that touch the diagonal or the candidate block.
#include "common.h"

namespace hstu {
namespace {

constexpr int DH = 128;            // bf16 head dim
constexpr int KT = kTileK;         // 64 keys per tile
constexpr int BQ = kBlockQ;        // 128 queries per block
constexpr int kBiasLen = BQ + KT;  // 191 distances per tile (padded)

__device__ __forceinline__ bool tile_visible_dev(int k0, int qa, int qe, int hist) {
  if (k0 < qe && qa < k0 + KT) return true;
  return k0 < hist && k0 < qe - 1;
}

// Key order inside each 32-key MFMA row block: MFMA row i reads key vperm(i)
// (bits 2 and 3 swapped), so that after S^T = K . Q^T the 8 score registers a
// lane feeds into one P . V k-step are 8 consecutive keys.
__device__ __forceinline__ int vperm(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}
// 16-byte-chunk XOR swizzles of the K and V tiles ([64 keys][128 dims] each).
// K: the 16 rows an A-operand read touches per cycle map to 16 chunk slots.
// V: the 4 rows x 2 chunks a 16-lane transposed read touches (and the other
// half-wave's 2 chunks) map to distinct slots.
__device__ __forceinline__ int kswz(int row) { return row & 15; }
__device__ __forceinline__ int vswz(int row) { return (row & 3) << 2; }

constexpr int kMaxPagesLds = kMaxItemPages;
constexpr int kMaxBuckets = 256;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ v4i16 lds_read_tr(const __attribute__((address_space(3))) uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Weights carry a factor log2(e): with y = log2(e) * x, the kernel forms
// y / (1 + 2^-y) = log2(e) * SiLU(x) (one FMA, one exp2, one add, one rcp,
// one multiply); the reduction multiplies by ln 2 to remove it.
constexpr float kLog2e = 1.44269504088896340736f;
__device__ __forceinline__ float silu_l2(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef const __attribute__((address_space(1))) void global_void;

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at
// dst + 16 l (dst is wave-uniform), without passing through registers.
__device__ __forceinline__ void dma16(const uint16_t* src, lds_u16* dst) {
  __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)dst, 16, 0, 0);
}

// The per-tile bias table is needed unless every query of the block sees the
// whole tile (no mask) at distances that fall in one bucket.
__device__ __forceinline__ bool needs_bias_table(int k0, int qa, int qe, int hist, int nb) {
  const int dlo = qa - (k0 + KT - 1), dhi = qe - 1 - k0;
  const bool unmasked = k0 + KT - 1 < qa && k0 + KT - 1 < hist;
  return !(unmasked && rel_bucket(dlo, nb) == rel_bucket(dhi, nb));
}

// K/V tiles are double-buffered in LDS: while the waves multiply tile t out
// of one buffer, the copy engine fills the other with the next visible tile,
// so each tile costs one barrier and no register staging.  The buffers are
// separate LDS objects and each loop half names its own, so the compiler can
// tell the in-flight copy does not touch the buffer being read.
template <bool PAGED>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnLaunch a) {
  __shared__ __attribute__((aligned(16))) uint16_t K0s[KT * DH];
  __shared__ __attribute__((aligned(16))) uint16_t V0s[KT * DH];
  __shared__ __attribute__((aligned(16))) uint16_t K1s[KT * DH];
  __shared__ __attribute__((aligned(16))) uint16_t V1s[KT * DH];
  lds_u16* const K0 = (lds_u16*)K0s;
  lds_u16* const V0 = (lds_u16*)V0s;
  lds_u16* const K1 = (lds_u16*)K1s;
  lds_u16* const V1 = (lds_u16*)V1s;
  __shared__ float bias0[256];          // log2(e) * bias, reversed distance order
  __shared__ float bias1[256];
  __shared__ float rab_s[kMaxBuckets];  // log2(e) * rab
  __shared__ int32_t pages_lds[PAGED ? kMaxPagesLds : 1];

  const uint64_t t_start = a.stamps ? __builtin_amdgcn_s_memrealtime() : 0;
  const WorkItem w = a.plan.items[blockIdx.x];
  if (w.slot < 0) return;  // padding entry of the dispatch order
  const int h = w.head;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = uniform(tid >> 6);
  const int wq0 = wave * 32;                 // first local query of this wave
  const bool wave_active = wq0 < w.count;
  const int qlocal = wq0 + l32;
  const int qpos = w.pos0 + qlocal;          // sequence position of this lane's query
  const int qa = w.pos0, qe = w.pos0 + w.count;
  const int hist = w.hist;
  const int nb = a.num_buckets;
  const int vis_lim = min(qpos, hist);       // keys below this are visible; so is key == qpos

  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);
  const uint16_t* kbase = static_cast<const uint16_t*>(PAGED ? a.k_pool : a.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(PAGED ? a.v_pool : a.v);

  // ---- stage the bias table and this work item's page-table slice ----
  for (int i = tid; i < nb; i += 256) rab_s[i] = a.rab[i] * kLog2e;
  const int P = PAGED ? a.plan.page_size : KT;
  const int p_shift = __ffs(P) - 1;          // the host guarantees a power of two >= 16
  int pg0 = 0;
  if (PAGED) {
    pg0 = (w.tile_begin * KT) >> p_shift;
    int pg1 = min((w.tile_end * KT + P - 1) >> p_shift, a.plan.max_pages);
    const int32_t* src = a.page_table + static_cast<int64_t>(w.user) * a.plan.max_pages + pg0;
    for (int i = tid; i < pg1 - pg0; i += 256) pages_lds[i] = src[i];
  }

  // Q^T as the B operand of S^T = K . Q^T: lane holds q[query l32][16 s + 8 g .. +8]
  bf16x8 qf[DH / 16];
  {
    const bool qv = qlocal < w.count;
    const uint16_t* qrow = qbase + static_cast<int64_t>(w.row0 + (qv ? qlocal : 0)) * a.q_stride + h * DH;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      u32x4 raw = qv ? *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * g) : u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 oacc[DH / 32];
#pragma unroll
  for (int t = 0; t < DH / 32; ++t) oacc[t] = f32x16{};

  // ---- tile copy: wave w fills rows 16 w .. 16 w + 15, four rows per
  // instruction; lane l of instruction i carries row 16 w + 4 i + l / 16,
  // LDS chunk slot l % 16, which holds global chunk slot ^ swizzle(row). ----
  const int lrow = lane >> 4, lslot = lane & 15;
  const int64_t row_stride = PAGED ? DH : a.kv_stride;
  int loffk[4], loffv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + lrow;  // row within the wave's 16 (swizzles only see row & 15)
    loffk[i] = static_cast<int>(r * row_stride) + 8 * (lslot ^ kswz(r));
    loffv[i] = static_cast<int>(r * row_stride) + 8 * (lslot ^ vswz(r));
  }
  // page of logical page lp of this user: from the staged slice, or (for the
  // first tile, copied before the slice is staged) from the table itself
  auto page_lds = [&](int lp) { return pages_lds[lp - pg0]; };
  auto page_glb = [&](int lp) {
    return a.page_table[static_cast<int64_t>(w.user) * a.plan.max_pages + lp];
  };
  auto copy_tile = [&](int tile, lds_u16* Kd, lds_u16* Vd, auto&& page_of) {
    const int k0 = tile * KT;
    const int r0 = k0 + 16 * wave;  // first key of this wave's rows
    if (r0 + 16 <= w.kv_len) {
      int64_t base;
      if (PAGED) {
        int page = uniform(page_of(r0 >> p_shift));
        page = (page >= 0 && page < a.num_pages) ? page : 0;
        base = a.pool_layer_offset + ((static_cast<int64_t>(page) * a.plan.H + h) * P + (r0 & (P - 1))) * DH;
      } else {
        base = static_cast<int64_t>(w.kv_row0 + r0) * a.kv_stride + h * DH;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dma16(kbase + base + loffk[i], Kd + (16 * wave + 4 * i) * DH);
        dma16(vbase + base + loffv[i], Vd + (16 * wave + 4 * i) * DH);
      }
    } else {
      // rows past the user's last key repeat that key: finite values whose
      // weights the mask zeroes
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + lrow;
        const int key = min(r0 + r, w.kv_len - 1);
        int64_t off;
        if (PAGED) {
          int page = page_of(key >> p_shift);
          page = (page >= 0 && page < a.num_pages) ? page : 0;
          off = a.pool_layer_offset + ((static_cast<int64_t>(page) * a.plan.H + h) * P + (key & (P - 1))) * DH;
        } else {
          off = static_cast<int64_t>(w.kv_row0 + key) * a.kv_stride + h * DH;
        }
        dma16(kbase + off + 8 * (lslot ^ kswz(r)), Kd + (16 * wave + 4 * i) * DH);
        dma16(vbase + off + 8 * (lslot ^ vswz(r)), Vd + (16 * wave + 4 * i) * DH);
      }
    }
  };
  // bias table of a tile, from the staged rab (or, for the first tile, filled
  // before rab is staged, from rab itself)
  auto fill_bias = [&](int tile, float* bias_rev, bool from_global) {
    const int k0 = tile * KT;
    if (needs_bias_table(k0, qa, qe, hist, nb) && tid < kBiasLen) {
      const int d = qa + BQ - 1 - k0 - tid;
      const int bk = rel_bucket(d, nb);
      bias_rev[tid] = d < 0 ? 0.f : (from_global ? a.rab[bk] * kLog2e : rab_s[bk]);
    }
  };
  // per-lane LDS read offsets (elements), hoisted out of the tile loop
  int kaddr[DH / 16];  // A operand of S^T: row vperm(l32) (+32 per row block), chunk (2s+g)
  {
    const int row = vperm(l32);
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) kaddr[s] = row * DH + 8 * ((2 * s + g) ^ kswz(row));
  }
  int vaddr[2][DH / 32];  // transposed B-operand reads of V
  {
    const int grp = lane >> 4, j = lane & 15;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 8 * g + 4 * r + (j >> 2);  // plus 16 ks (does not change the swizzle)
      const int dcol = 16 * (grp & 1) + 4 * (j & 3);
#pragma unroll
      for (int nt = 0; nt < DH / 32; ++nt) {
        int d = 32 * nt + dcol;
        vaddr[r][nt] = row * DH + 8 * ((d >> 3) ^ vswz(row)) + (d & 7);
      }
    }
  }

  auto compute_tile = [&](int t, const lds_u16* Ks, const lds_u16* Vs, const float* bias_rev) {
    const int k0 = t * KT;
    // ---- S^T = K . Q^T (register r of block mt: key 32 mt + 16 (r/8) + 8 g + r%8) ----
    f32x16 sacc[KT / 32];
#pragma unroll
    for (int mt = 0; mt < KT / 32; ++mt) {
      sacc[mt] = f32x16{};
#pragma unroll
      for (int s = 0; s < DH / 16; ++s) {
        bf16x8 kf = *(const __attribute__((address_space(3))) bf16x8*)(&Ks[kaddr[s] + 32 * mt * DH]);
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[mt], 0, 0, 0);
      }
    }

    // ---- bias, mask, SiLU: weights y / (1 + 2^-y) with y = log2(e) (q.k + bias) ----
    const int wq_lo = qa + wq0, wq_hi = min(qa + wq0 + 31, qe - 1);
    const int dmin = wq_lo - (k0 + KT - 1), dmax = wq_hi - k0;
    const bool full = (k0 + KT - 1 < wq_lo) && (k0 + KT - 1 < hist);  // no masking needed
    const bool uni = dmin >= 0 && rel_bucket(dmin, nb) == rel_bucket(dmax, nb);
    const int kbase_lane = k0 + 8 * g;
    // three cases, in falling order of frequency: far tiles with one bias
    // value, far tiles spanning bucket edges (bias table, no mask), and tiles
    // on the diagonal or the candidate block (bias table and mask)
    const float* brow = &bias_rev[BQ - 1 - qlocal + 8 * g];
    if (full && uni) {
      const float ub = rab_s[rel_bucket(dmax, nb)];
#pragma unroll
      for (int mt = 0; mt < KT / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[mt][r] = silu_l2(fmaf(sacc[mt][r], kLog2e, ub));
    } else if (full) {
#pragma unroll
      for (int mt = 0; mt < KT / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int koff = 32 * mt + 16 * (r >> 3) + (r & 7);
          sacc[mt][r] = silu_l2(fmaf(sacc[mt][r], kLog2e, brow[koff]));
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < KT / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int koff = 32 * mt + 16 * (r >> 3) + (r & 7);
          const int key = kbase_lane + koff;
          const float p = silu_l2(fmaf(sacc[mt][r], kLog2e, brow[koff]));
          sacc[mt][r] = (key < vis_lim || key == qpos) ? p : 0.f;
        }
    }

    // ---- O += P . V (V read transposed from its row-major tile) ----
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      const f32x16& src = sacc[ks >> 1];
      const int base = 8 * (ks & 1);
      bf16x8 pa;
#pragma unroll
      for (int e = 0; e < 8; ++e) pa[e] = static_cast<__bf16>(src[base + e]);
#pragma unroll
      for (int nt = 0; nt < DH / 32; ++nt) {
        // assembled from whole dwords: extracting the 16-bit elements of the
        // transposed reads one by one is lowered incorrectly by this compiler
        u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr(&Vs[vaddr[0][nt] + 16 * ks * DH]));
        u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr(&Vs[vaddr[1][nt] + 16 * ks * DH]));
        bf16x8 vb = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        oacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vb, oacc[nt], 0, 0, 0);
      }
    }
  };

  auto visible_tile = [&](int t) { return tile_visible_dev(t * KT, qa, qe, hist); };
  auto next_visible = [&](int t) {
    ++t;
    while (t < w.tile_end && !visible_tile(t)) ++t;
    return t;
  };
  // the first tile's copy and bias go out with the rest of the set-up loads
  int t = w.tile_begin;
  while (t < w.tile_end && !visible_tile(t)) ++t;
  if (t < w.tile_end) {
    fill_bias(t, bias0, true);
    copy_tile(t, K0, V0, page_glb);
  }
  __syncthreads();  // rab, page-table slice and tile t staged
  const uint64_t t_setup = a.stamps ? __builtin_amdgcn_s_memrealtime() : 0;

  // two tiles per trip so that each half names its buffers statically
  while (t < w.tile_end) {
    int tn = next_visible(t);
    if (tn < w.tile_end) {
      fill_bias(tn, bias1, false);
      copy_tile(tn, K1, V1, page_lds);
    }
    __builtin_amdgcn_sched_barrier(0);  // issue the copy before the tile's LDS reads
    if (wave_active) compute_tile(t, K0, V0, bias0);
    __syncthreads();  // buffer 1 filled; buffer 0 free
    if (tn >= w.tile_end) break;
    t = tn;
    tn = next_visible(t);
    if (tn < w.tile_end) {
      fill_bias(tn, bias0, false);
      copy_tile(tn, K0, V0, page_lds);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (wave_active) compute_tile(t, K1, V1, bias1);
    __syncthreads();  // buffer 0 filled; buffer 1 free
    t = tn;
  }

  const uint64_t t_loop = a.stamps ? __builtin_amdgcn_s_memrealtime() : 0;
  // ---- partial tile [BQ][DH] fp32 (times log2 e).  A lane holds column
  // 32 nt + l32 of rows 8(r/4)+4g+r%4; the tile goes through LDS (the four
  // K/V buffers, free after the last barrier, 32 rows each) so that whole
  // 512-byte rows leave in 16-byte stores ----
  auto stage_row = [&](int row) -> __attribute__((address_space(3))) float* {
    lds_u16* b = row < 32 ? K0 : row < 64 ? V0 : row < 96 ? K1 : V1;
    return (__attribute__((address_space(3))) float*)(b) + (row & 31) * DH;
  };
  if (wave_active) {
#pragma unroll
    for (int nt = 0; nt < DH / 32; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wq0 + 8 * (r >> 2) + 4 * g + (r & 3);
        stage_row(row)[32 * nt + l32] = oacc[nt][r];
      }
  }
  __syncthreads();
  float* out = static_cast<float*>(a.partials) + static_cast<int64_t>(w.slot) * BQ * DH;
  const int srow = lane >> 5, sch = lane & 31;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int row = wq0 + 2 * it + srow;
    if (row < w.count)
      *reinterpret_cast<f32x4*>(out + row * DH + 4 * sch) =
          *(const __attribute__((address_space(3))) f32x4*)(stage_row(row) + 4 * sch);
  }
  if (a.stamps && tid == 0) {
    AttnStamp st;
    st.start = t_start;
    st.setup_done = t_setup;
    st.loop_done = t_loop;
    st.end = __builtin_amdgcn_s_memrealtime();
    st.hw_id = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_ID, all 32 bits
    st.xcc_id = __builtin_amdgcn_s_getreg((3 << 11) | 20);   // XCC_ID[3:0]
    st.slot = w.slot;
    st.tiles = w.tile_end - w.tile_begin;
    a.stamps[blockIdx.x] = st;
  }
}

// ---------------------------------------------------------------------------
// fp32: one thread per query, keys staged 32 at a time, exact bucket per pair
// ---------------------------------------------------------------------------
template <int D, bool PAGED>
__global__ __launch_bounds__(128) void attn_f32_kernel(AttnLaunch a) {
  constexpr int SK = 32;
  __shared__ float Ks[SK][D + 1];
  __shared__ float Vs[SK][D + 1];
  const WorkItem w = a.plan.items[blockIdx.x];
  if (w.slot < 0) return;  // padding entry of the dispatch order
  const int h = w.head, tid = threadIdx.x;
  const int qpos = w.pos0 + tid;
  const bool qv = tid < w.count;
  const float* qbase = static_cast<const float*>(a.q);
  const float* kbase = static_cast<const float*>(PAGED ? a.k_pool : a.k);
  const float* vbase = static_cast<const float*>(PAGED ? a.v_pool : a.v);
  float q[D], o[D];
  for (int e = 0; e < D; ++e) {
    q[e] = qv ? qbase[static_cast<int64_t>(w.row0 + tid) * a.q_stride + h * D + e] : 0.f;
    o[e] = 0.f;
  }
  const int qa = w.pos0, qe = w.pos0 + w.count;
  for (int tile = w.tile_begin; tile < w.tile_end; ++tile) {
    if (!tile_visible_dev(tile * KT, qa, qe, w.hist)) continue;
    for (int sub = 0; sub < KT; sub += SK) {
      const int k0 = tile * KT + sub;
      __syncthreads();
      for (int i = tid; i < SK * D; i += 128) {
        int kk = i / D, e = i % D, j = k0 + kk;
        const float* kr = nullptr;
        const float* vr = nullptr;
        if (j < w.kv_len) {
          if (PAGED) {
            const int P = a.plan.page_size;
            int lp = j / P;
            int page = lp < a.plan.max_pages
                           ? a.page_table[static_cast<int64_t>(w.user) * a.plan.max_pages + lp]
                           : -1;
            if (page >= 0 && page < a.num_pages) {
              int64_t off = a.pool_layer_offset +
                            ((static_cast<int64_t>(page) * a.plan.H + h) * P + (j % P)) * D;
              kr = kbase + off;
              vr = vbase + off;
            }
          } else {
            kr = kbase + static_cast<int64_t>(w.kv_row0 + j) * a.kv_stride + h * D;
            vr = vbase + static_cast<int64_t>(w.kv_row0 + j) * a.kv_stride + h * D;
          }
        }
        Ks[kk][e] = kr ? kr[e] : 0.f;
        Vs[kk][e] = vr ? vr[e] : 0.f;
      }
      __syncthreads();
      if (!qv) continue;
      for (int kk = 0; kk < SK; ++kk) {
        const int j = k0 + kk;
        const bool vis = (j == qpos) || (j < qpos && j < w.hist);
        if (!vis) continue;
        float s = 0.f;
        for (int e = 0; e < D; ++e) s += q[e] * Ks[kk][e];
        s += a.rab[rel_bucket(qpos - j, a.num_buckets)];
        const float p = s / (1.0f + expf(-s));
        for (int e = 0; e < D; ++e) o[e] += p * Vs[kk][e];
      }
    }
  }
  if (!qv) return;
  float* out = static_cast<float*>(a.partials) + (static_cast<int64_t>(w.slot) * BQ + tid) * D;
  for (int e = 0; e < D; ++e) out[e] = o[e];
}

template <bool PAGED>
hipError_t launch_f32(const AttnLaunch& a, hipStream_t s) {
  dim3 grid(a.plan.n_items);
  switch (a.plan.dh) {
    case 32: hipLaunchKernelGGL((attn_f32_kernel<32, PAGED>), grid, dim3(128), 0, s, a); break;
    case 64: hipLaunchKernelGGL((attn_f32_kernel<64, PAGED>), grid, dim3(128), 0, s, a); break;
    case 128: hipLaunchKernelGGL((attn_f32_kernel<128, PAGED>), grid, dim3(128), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnLaunch& a, hipStream_t s) {
  if (a.plan.n_items == 0) return hipSuccess;
  const bool paged = a.plan.page_size > 0;
  if (a.dtype == HSTU_BF16) {
    if (a.plan.dh != DH) return hipErrorInvalidValue;
    dim3 grid(a.plan.n_items);
    if (paged) hipLaunchKernelGGL(attn_bf16_kernel<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(attn_bf16_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return paged ? launch_f32<true>(a, s) : launch_f32<false>(a, s);
}

}  // namespace hstu

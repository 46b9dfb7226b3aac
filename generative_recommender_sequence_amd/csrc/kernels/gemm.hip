// The two projections of the HSTU layer ("How Generative Recommenders Are
// Redefining RecSys at Scale", section HSTU):
//   f1: [U|V|Q|K] = SiLU(LayerNorm(x) . W1)   (epilogue 0)
//   f2: y = x + g . W2                        (epilogue 1)
// A is row-major [M][K]; the weights come output-major, Wt [N][K] (the
// transpose of the x . W layout), so both operands are rows of contiguous k.
//
// bf16 kernel: a BM x BN output tile per 256-thread block (4 waves as 2 x 2,
// each wave (BM/2) x (BN/2) as v_mfma_f32_32x32x16_bf16 tiles), K in steps of
// 64.  Both operand tiles are double-buffered in LDS and filled by direct
// global -> LDS copies (no register staging, one barrier per k step); rows are
// 64 k wide with a 16-byte-chunk XOR swizzle that keeps the 16-lane operand
// reads free of bank conflicts.  Each MFMA multiplies a Wt fragment by an x
// fragment, producing C^T tiles, so a lane owns 4 consecutive output columns
// of one row (and reads the residual 8 bytes at a time).  The finished tile
// goes through LDS (the freed operand buffers) so that whole 256-byte rows
// leave in 16-byte stores.  Blocks are dealt to the 8 XCDs so that the n
// tiles of one m tile share an L2.
//
// Epilogue 0 applies the pre-norm algebraically: with mu, rstd the row
// statistics of x and s_n = sum_k W1[k][n] (computed once per weight set),
//     LayerNorm(x) . W1 = rstd * (x . W1 - mu * s_n),
// so x is multiplied as stored (no normalised copy).  The statistics come as
// per-share (mean, sum of squared deviations) slots, combined per row.  The
// SiLU'd columns are routed by chunk: U and Q to the token-major buffer, K and
// V either to the same buffer (contiguous keys) or straight into their pages
// (paged cache; the append of the new tokens), at each row's pool slot, which
// the row-statistics kernel of the stack's first layer looks up once for all
// layers.
//
// Epilogue 1 may also leave the statistics of its output rows for the next
// layer's pre-norm: per row and 128-column tile, the mean and the sum of
// squared deviations of the stored (bf16-rounded) values, two-pass over the
// registers, added across the two column waves in fixed order.
//
// Epilogue 2 is the multitask ranking head's hidden layer and output dot
// product: A's rows are gathered through a row list, each column n gets
// ReLU(acc + b[n]) * w[n], and the block sums its BN columns per row into one
// partial logit; a small kernel adds a task's partials and its output bias.
//
// fp32: plain 64 x 64-tile FMA kernels, with the pre-norm done by a separate
// row LayerNorm and the append by the copy kernel.
#include "common.h"

namespace hstu {
namespace {

constexpr int GBK = 64;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef const __attribute__((address_space(1))) void global_void;

__device__ __forceinline__ void dma16(const uint16_t* src, lds_u16* dst) {
  __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)dst, 16, 0, 0);
}

// two floats to a pair of bf16 (round to nearest even) in one conversion
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v{lo, hi}), bf16x2v));
}

// 16-byte chunk slot of logical chunk c in row r of a 64-wide tile (rows are
// 128 B, two per 64 banks): 16 consecutive rows read at one logical chunk hit
// 16 distinct bank groups.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// Routing of f1's output columns (epilogue 0).
struct F1Route {
  const RowStat* stats;       // [M][stat_slots] statistics of the input rows
  int32_t stat_slots;         // 1 .. kMaxStatSlots, dividing K
  float eps;
  const int64_t* row_slots;   // [M] pool slot of each row, or -1 (with k_pool)
  const float* colsum;        // [N] column sums of W1
  uint16_t* uvqk;             // [M][4 inner] token-major destination
  int32_t inner;              // H * dh
  bool kv_to_uvqk;            // also write the K and V chunks to uvqk
  uint16_t* k_pool;           // paged K/V destination (nullptr: none)
  uint16_t* v_pool;
  int64_t pool_layer_offset;  // elements
  int32_t dh, page_size;
  // epilogue 2 (head)
  const int32_t* a_rows;      // [M]: the row of A that output row m reads
  int32_t a_rows_max;         // rows of A; indices are clamped to [0, a_rows_max)
  const float* h_bias;        // [N] hidden bias
  const float* h_wout;        // [N] output weights
  float* h_partial;           // [M][N / BN] partial logits
  uint16_t* s_out;            // epilogue 0: the pre-activation x^ W1 [M][N] (nullptr: not kept)
  RowStat* y_stats;           // epilogue 1: [M][N / BN] statistics of C's rows (nullptr: not kept)
};

// NK > 0 (64-row tiles, K = 64 NK): the k loop fully unrolled over three LDS
// stages, copies issued two steps ahead, each step waiting only for its own
// stage's copies (an exact wait count and a bare barrier, so the next
// stage's copies stay in flight); NK = 0: two stages, one step ahead.
template <int BM, int BN, int EPI, int NK = 0>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ Wt,
                                                           uint16_t* __restrict__ C,
                                                           const uint16_t* __restrict__ R,
                                                           F1Route route, int32_t M, int32_t N,
                                                           int32_t K) {
  constexpr int MT = BM / 64, NT = BN / 64;  // 32-wide MFMA tiles per wave along m, n
  __shared__ __attribute__((aligned(16))) uint16_t A0s[BM * GBK];
  __shared__ __attribute__((aligned(16))) uint16_t A1s[BM * GBK];
  __shared__ __attribute__((aligned(16))) uint16_t B0s[BN * GBK];
  __shared__ __attribute__((aligned(16))) uint16_t B1s[BN * GBK];
  lds_u16* const A0 = (lds_u16*)A0s;
  lds_u16* const A1 = (lds_u16*)A1s;
  lds_u16* const B0 = (lds_u16*)B0s;
  lds_u16* const B1 = (lds_u16*)B1s;
  constexpr bool kThree = NK > 0;
  static_assert(!kThree || BM == 64, "three stages fit two blocks a CU only with 64-row tiles");
  __shared__ __attribute__((aligned(16))) uint16_t A2s[kThree ? BM * GBK : 8];
  __shared__ __attribute__((aligned(16))) uint16_t B2s[kThree ? BN * GBK : 8];
  lds_u16* const A2 = (lds_u16*)A2s;
  lds_u16* const B2 = (lds_u16*)B2s;

  // XCD-aware tile order: block b runs on XCD b % 8 (the grid is a multiple
  // of 8); XCD x takes tiles x * per_xcd .. , n fastest.
  const int n_tiles_n = N / BN;
  const int tiles = ((M + BM - 1) / BM) * n_tiles_n;
  const int per_xcd = gridDim.x / 8;
  const int id = static_cast<int>(blockIdx.x % 8) * per_xcd + static_cast<int>(blockIdx.x / 8);
  if (id >= tiles) return;
  const int m0 = (id / n_tiles_n) * BM;
  const int n0 = (id % n_tiles_n) * BN;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

  // copy: instruction j of the block fills rows 8 j .. 8 j + 7 (1 KB); lane l
  // carries row 8 j + l / 8, chunk slot l % 8, i.e. logical chunk slot ^ swz8(row)
  const int crow = lane >> 3, cslot = lane & 7;
  int64_t a_src[BM / 32];  // epilogue 2: gathered source rows, looked up once
  if (EPI == 2) {
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
      const int src = route.a_rows[min(m0 + 8 * (wave + 4 * i) + crow, M - 1)];
      a_src[i] = static_cast<int64_t>(min(max(src, 0), route.a_rows_max - 1)) * K;
    }
  }
  auto copy_k = [&](int k0, lds_u16* Ad, lds_u16* Bd) {
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
      const int r = 8 * (wave + 4 * i) + crow;
      const int m = min(m0 + r, M - 1);  // rows past M repeat the last row
      const int64_t row_off = EPI == 2 ? a_src[i] : static_cast<int64_t>(m) * K;
      dma16(A + row_off + k0 + 8 * (cslot ^ swz8(r)), Ad + 8 * (wave + 4 * i) * GBK);
    }
#pragma unroll
    for (int i = 0; i < BN / 32; ++i) {
      const int r = 8 * (wave + 4 * i) + crow;
      dma16(Wt + static_cast<int64_t>(n0 + r) * K + k0 + 8 * (cslot ^ swz8(r)), Bd + 8 * (wave + 4 * i) * GBK);
    }
  };

  // operand reads: row (wave half) + 32 t + l32, logical chunk 2 ks + g; the
  // swizzle only sees l32 (the other row terms are multiples of 16)
  int koff[GBK / 16];
#pragma unroll
  for (int ks = 0; ks < GBK / 16; ++ks) koff[ks] = l32 * GBK + 8 * ((2 * ks + g) ^ swz8(l32));
  const int a_row0 = wm * (BM / 2) * GBK, b_row0 = wn * (BN / 2) * GBK;

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16{};

  auto mma_k = [&](const lds_u16* As, const lds_u16* Bs) {
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      bf16x8 af[MT], bfr[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        af[i] = *(const __attribute__((address_space(3))) bf16x8*)(&As[a_row0 + 32 * i * GBK + koff[ks]]);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        bfr[j] = *(const __attribute__((address_space(3))) bf16x8*)(&Bs[b_row0 + 32 * j * GBK + koff[ks]]);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)  // C^T tile: rows n, columns m
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  };

  // epilogue inputs fetched up front so that their latency hides under the
  // k loop: each lane's row statistics and pool slots (f1) or residual
  // values (f2), and the block's column sums (f1, into LDS)
  __shared__ __attribute__((aligned(16))) float cs_lds[EPI == 0 ? BN : 4];
  __shared__ __attribute__((aligned(16))) float hb_lds[EPI == 2 ? BN : 4];
  __shared__ __attribute__((aligned(16))) float hw_lds[EPI == 2 ? BN : 4];
  RowStat rstat[MT][kMaxStatSlots];
  int64_t slot[MT];
  f32x4 cs_val;
  u32x2 resid[MT][NT][4];
  if (EPI == 2) {
    if (tid < BN / 4) {
      *reinterpret_cast<f32x4*>(&hb_lds[4 * tid]) = *reinterpret_cast<const f32x4*>(&route.h_bias[n0 + 4 * tid]);
      *reinterpret_cast<f32x4*>(&hw_lds[4 * tid]) = *reinterpret_cast<const f32x4*>(&route.h_wout[n0 + 4 * tid]);
    }
  } else if (EPI == 0) {
    // column sums: loaded here, stored to LDS after the first k step's copy is issued
    cs_val = tid < BN / 4 ? *reinterpret_cast<const f32x4*>(&route.colsum[n0 + 4 * tid]) : f32x4{};
    // straight-line loads (slots past stat_slots re-read the last one), so
    // that none of them is waited for before the k loop's first barrier
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = min(m0 + wm * (BM / 2) + 32 * i + l32, M - 1);
      const RowStat* sp = route.stats + static_cast<int64_t>(m) * route.stat_slots;
#pragma unroll
      for (int t = 0; t < kMaxStatSlots; ++t) rstat[i][t] = sp[min(t, route.stat_slots - 1)];
      slot[i] = route.k_pool ? route.row_slots[m] : -1;
    }
  } else if (EPI == 1) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = min(m0 + wm * (BM / 2) + 32 * i + l32, M - 1);
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          resid[i][j][q] = *reinterpret_cast<const u32x2*>(R + static_cast<int64_t>(m) * N + n0 + wn * (BN / 2) +
                                                           32 * j + 8 * q + 4 * g);
    }
  }

  const int nk = kThree ? NK : K / GBK;
  copy_k(0, A0, B0);
  if (kThree) copy_k(GBK, A1, B1);
  if (EPI == 0 && tid < BN / 4) *reinterpret_cast<f32x4*>(&cs_lds[4 * tid]) = cs_val;
  if (!kThree) __syncthreads();  // k step 0 in buffer 0 (and the prefetched row statistics in)
  // f1: each lane's row statistics
  float mu[MT], rstd[MT];
  if (EPI == 0) {
    const float inv_slots = 1.0f / route.stat_slots, share = static_cast<float>(K) * inv_slots;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      float mean = 0.f;
#pragma unroll
      for (int t = 0; t < kMaxStatSlots; ++t) mean += t < route.stat_slots ? rstat[i][t].mean : 0.f;
      mean *= inv_slots;
      float m2 = 0.f, dev = 0.f;
#pragma unroll
      for (int t = 0; t < kMaxStatSlots; ++t) {
        const float dm = rstat[i][t].mean - mean;
        m2 += t < route.stat_slots ? rstat[i][t].m2 : 0.f;
        dev += t < route.stat_slots ? dm * dm : 0.f;
      }
      mu[i] = mean;
      rstd[i] = __builtin_amdgcn_rsqf((m2 + share * dev) * (1.0f / K) + route.eps);
    }
  }
  if constexpr (kThree) {
    // copy instructions a wave issues per stage
    constexpr int kDma = BM / 32 + BN / 32;
    lds_u16* const As[3] = {A0, A1, A2};
    lds_u16* const Bs[3] = {B0, B1, B2};
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      // this wave's copies of step kt have landed (those of step kt + 1 may
      // still be in flight; vmcnt counts in issue order), then every wave's
      // have, and every wave is done with step kt - 1, whose buffer the
      // copies of step kt + 2 refill
      if (kt + 1 < NK)
        __builtin_amdgcn_s_waitcnt(0x0070 | (kDma & 15) | ((kDma >> 4) << 14));  // vmcnt(kDma), lgkmcnt(0)
      else
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      if (kt + 2 < NK) copy_k((kt + 2) * GBK, As[(kt + 2) % 3], Bs[(kt + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);  // issue the copies before this step's reads
      mma_k(As[kt % 3], Bs[kt % 3]);
    }
    __syncthreads();  // every wave done with the operand buffers the epilogue reuses
  }
  for (int kt = 0; !kThree && kt < nk; kt += 2) {
    if (kt + 1 < nk) copy_k((kt + 1) * GBK, A1, B1);
    __builtin_amdgcn_sched_barrier(0);  // issue the copy before this step's reads
    mma_k(A0, B0);
    __syncthreads();  // buffer 1 filled; buffer 0 free
    if (kt + 1 >= nk) break;
    if (kt + 2 < nk) copy_k((kt + 2) * GBK, A0, B0);
    __builtin_amdgcn_sched_barrier(0);
    mma_k(A1, B1);
    __syncthreads();  // buffer 0 filled; buffer 1 free
  }

  if (EPI == 2) {
    // each lane sums ReLU(acc + b) * w over its 16 NT columns of row l32; the
    // two lane halves and then the two column waves are added in fixed order
    __shared__ float red[2][BM];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn * (BN / 2) + 32 * j + 8 * q + 4 * g;
          const f32x4 hb = *reinterpret_cast<const f32x4*>(&hb_lds[nl]);
          const f32x4 hw = *reinterpret_cast<const f32x4*>(&hw_lds[nl]);
#pragma unroll
          for (int e = 0; e < 4; ++e) sum += fmaxf(acc[i][j][4 * q + e] + hb[e], 0.f) * hw[e];
        }
      sum += __shfl_xor(sum, 32);
      if (g == 0) red[wn][wm * (BM / 2) + 32 * i + l32] = sum;
    }
    __syncthreads();
    if (tid < BM && m0 + tid < M)
      route.h_partial[static_cast<int64_t>(m0 + tid) * (N / BN) + n0 / BN] = red[0][tid] + red[1][tid];
    return;
  }

  // epilogue, phase 1: each lane finishes its values (row m = ... + l32,
  // columns n = ... + 8 (r/4) + 4 g + [0, 4)) and writes them as bf16 into an
  // LDS image of the output tile, in the operand buffers the k loop has
  // released: rows 0-63 in A0 and 64-127 in B0 (BM = 128), all rows in B0
  // (BM = 64).  The 16-byte chunk c of local row r sits at slot c ^ (r & 15).
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  auto stage_row = [&](int r) -> lds_u16* {
    if (BM == 128) return r < 64 ? A0 + r * BN : B0 + (r - 64) * BN;
    return B0 + r * BN;
  };
  __shared__ int64_t slot_lds[EPI == 0 ? BM : 1];  // pool offset of each local row, or -1
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int rl = wm * (BM / 2) + 32 * i + l32;
    const int m = m0 + rl;
    if (m >= M) continue;
    if (EPI == 0 && wn == 0 && g == 0)
      slot_lds[rl] = route.k_pool && slot[i] >= 0 ? route.pool_layer_offset + slot[i] : -1;
    lds_u16* const srow = stage_row(rl);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * (BN / 2) + 32 * j + 8 * q + 4 * g;  // first of this lane's 4 columns
        float v[4], z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
        if (EPI == 0) {
          const f32x4 cs = *reinterpret_cast<const f32x4*>(&cs_lds[nl]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            z[e] = rstd[i] * (v[e] - mu[i] * cs[e]);
            v[e] = z[e] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z[e] * -1.44269504088896340736f));
          }
        } else if (EPI == 1) {
          const u32x2 r2 = resid[i][j][q];
          v[0] += bf2f(r2[0] & 0xFFFFu);
          v[1] += bf2f(r2[0] >> 16);
          v[2] += bf2f(r2[1] & 0xFFFFu);
          v[3] += bf2f(r2[1] >> 16);
        }
        const u32x2 packed = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        if (EPI == 1) {  // the stored values, for the row statistics
          acc[i][j][4 * q + 0] = bf2f(packed[0] & 0xFFFFu);
          acc[i][j][4 * q + 1] = bf2f(packed[0] >> 16);
          acc[i][j][4 * q + 2] = bf2f(packed[1] & 0xFFFFu);
          acc[i][j][4 * q + 3] = bf2f(packed[1] >> 16);
        }
        if (EPI == 0 && route.s_out) {  // pre-activation tap (f1), stored directly
          const u32x2 pre = {pack_bf16(z[0], z[1]), pack_bf16(z[2], z[3])};
          *reinterpret_cast<u32x2*>(route.s_out + static_cast<int64_t>(m) * N + n0 + nl) = pre;
        }
        *(lds_u32x2*)(srow + 8 * ((nl >> 3) ^ (rl & 15)) + 4 * g) = packed;
      }
    }
  }
  __syncthreads();

  // phase 2: whole rows out, 4 rows an instruction (16 lanes x 16 bytes a
  // row).  A tile is one head of one chunk of [U|V|Q|K] (f1 checks that the
  // tile width is the head size), so its routing is block-uniform.
  {
    const int crow = lane >> 4, cch = lane & 15;
    constexpr int RPW = BM / 4;  // rows per wave
    int chunk = 0, h = 0;
    if (EPI == 0) {
      chunk = n0 / route.inner;  // 0 U, 1 V, 2 Q, 3 K
      h = (n0 - chunk * route.inner) / route.dh;
    }
    const bool is_kv = EPI == 0 && route.k_pool && (chunk == 1 || chunk == 3);
    const bool to_uvqk = EPI == 0 && (!is_kv || route.kv_to_uvqk);
    uint16_t* const pool = chunk == 3 ? route.k_pool : route.v_pool;
    const int64_t head_off = static_cast<int64_t>(h) * route.page_size * route.dh;
#pragma unroll
    for (int it = 0; it < RPW / 4; ++it) {
      const int rl = wave * RPW + 4 * it + crow;
      const int m = m0 + rl;
      if (m >= M) continue;
      const u32x4 val = *(const lds_u32x4*)(stage_row(rl) + 8 * (cch ^ (rl & 15)));
      if (EPI == 1 || EPI == 3) {
        *reinterpret_cast<u32x4*>(C + static_cast<int64_t>(m) * N + n0 + 8 * cch) = val;
        continue;
      }
      // f1's output streams past the L2 (non-temporal): it is not re-read by
      // this launch, and evicting W1 and the x rows for it cost more
      if (to_uvqk)
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(route.uvqk + static_cast<int64_t>(m) * N + n0 + 8 * cch));
      if (is_kv) {
        const int64_t pr = slot_lds[rl];
        if (pr >= 0) __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(pool + pr + head_off + 8 * cch));
      }
    }
  }

  if (EPI == 1 && route.y_stats) {
    // the row's 128 tile values: 2 x 32 per wave (lane halves g), two waves (wn)
    __shared__ float part[2][2][EPI == 1 ? BM : 1];
    float mean_t[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][j][e];
      s += __shfl_xor(s, 32);
      if (g == 0) part[0][wn][wm * (BM / 2) + 32 * i + l32] = s;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int rl = wm * (BM / 2) + 32 * i + l32;
      mean_t[i] = (part[0][0][rl] + part[0][1][rl]) * (1.0f / BN);
      float q2 = 0.f;
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float dv = acc[i][j][e] - mean_t[i];
          q2 += dv * dv;
        }
      q2 += __shfl_xor(q2, 32);
      if (g == 0) part[1][wn][rl] = q2;
    }
    __syncthreads();
    if (tid < BM && m0 + tid < M)
      route.y_stats[static_cast<int64_t>(m0 + tid) * (N / BN) + n0 / BN] =
          RowStat{(part[0][0][tid] + part[0][1][tid]) * (1.0f / BN), part[1][0][tid] + part[1][1][tid]};
  }
}

// Per-row (mean, sum of squared deviations) of x, two-pass from registers,
// one row a wave, kStatWaves waves a block.  Blocks past the rows' blocks sum
// the rows of Wt (the column sums of W1 that the f1 epilogue needs) unless the
// caller supplies them.
constexpr int kStatWaves = 4;
template <int kMaxChunks>  // cols <= 64 * 8 * kMaxChunks
__global__ __launch_bounds__(64 * kStatWaves) void row_stats_kernel(const uint16_t* __restrict__ x,
                                                                    RowStat* __restrict__ stats,
                                                                    int32_t rows, int32_t cols,
                                                                    const uint16_t* __restrict__ wt,
                                                                    float* __restrict__ colsum,
                                                                    int32_t wt_rows, RowSlots sl) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int stat_blocks = (rows + kStatWaves - 1) / kStatWaves;
  const bool is_wt = static_cast<int>(blockIdx.x) >= stat_blocks;
  const int r = (is_wt ? static_cast<int>(blockIdx.x) - stat_blocks : static_cast<int>(blockIdx.x)) * kStatWaves + wave;
  if (r >= (is_wt ? wt_rows : rows)) return;
  const uint16_t* src = (is_wt ? wt : x) + static_cast<int64_t>(r) * cols;
  u32x4 raw[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int col = 8 * (lane + 64 * c);
    raw[c] = col < cols ? *reinterpret_cast<const u32x4*>(src + col) : u32x4{0u, 0u, 0u, 0u};
  }
  if (!is_wt && sl.out && lane == 0) {
    // the row's page slot: its (user, position), then the page table
    const RowPos rp = sl.row_pos[r];
    const int lp = rp.pos / sl.page_size;
    int64_t off = -1;
    if (lp < sl.max_pages) {
      const int page = sl.page_table[static_cast<int64_t>(rp.user) * sl.max_pages + lp];
      if (page >= 0 && page < sl.num_pages)
        off = (static_cast<int64_t>(page) * sl.H * sl.page_size + (rp.pos - lp * sl.page_size)) * sl.dh;
    }
    sl.out[r] = off;
  }
  float v[kMaxChunks * 8];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[8 * c + e] = bf2f(static_cast<uint16_t>((e & 1) ? (raw[c][e >> 1] >> 16) : (raw[c][e >> 1] & 0xFFFFu)));
      s += v[8 * c + e];
    }
  s = wave_sum(s);
  if (is_wt) {
    if (lane == 0) colsum[r] = s;
    return;
  }
  const float mean = s / cols;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (8 * (lane + 64 * c) < cols) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dv = v[8 * c + e] - mean;
        q += dv * dv;
      }
    }
  }
  q = wave_sum(q);
  if (lane == 0) stats[r] = RowStat{mean, q};
}

constexpr int FT = 64, FK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ Bm,
                                                       float* __restrict__ C,
                                                       const float* __restrict__ R, int32_t M,
                                                       int32_t N, int32_t K) {
  __shared__ float As[FK][FT + 1];
  __shared__ float Bs[FK][FT + 1];
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int m0 = blockIdx.y * FT, n0 = blockIdx.x * FT;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FK) {
    for (int i = threadIdx.x; i < FK * FT; i += 256) {
      int kk = i % FK, mm = i / FK;
      int m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < M && k < K) ? A[static_cast<int64_t>(m) * K + k] : 0.f;
      int nn = i % FT, kb = i / FT;
      int n = n0 + nn, k2 = k0 + kb;
      Bs[kb][nn] = (n < N && k2 < K) ? Bm[static_cast<int64_t>(n) * K + k2] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < FK; ++kk)
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] += As[kk][ty + 16 * i] * Bs[kk][tx + 16 * j];
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      int m = m0 + ty + 16 * i, n = n0 + tx + 16 * j;
      if (m < M && n < N) {
        int64_t idx = static_cast<int64_t>(m) * N + n;
        float v = acc[i][j];
        if (EPI == 0) v = v / (1.0f + expf(-v));
        else v += R[idx];
        C[idx] = v;
      }
    }
}

// logits[m][t] = c[t] + the task's partials (in column order)
__global__ __launch_bounds__(256) void head_finalize_kernel(const float* __restrict__ partial,
                                                           int32_t per_task, int32_t tasks,
                                                           const float* __restrict__ c,
                                                           float* __restrict__ logits, int32_t M) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(M) * tasks) return;
  const int t = static_cast<int>(idx % tasks);
  const float* p = partial + idx * per_task;
  float z = c[t];
  for (int k = 0; k < per_task; ++k) z += p[k];
  logits[idx] = z;
}

}  // namespace

hipError_t launch_row_stats(const void* x, RowStat* stats, int32_t rows, int32_t cols, const void* w1t,
                            float* colsum, int32_t w1t_rows, const RowSlots& sl, hipStream_t s) {
  if (rows == 0 && w1t_rows == 0) return hipSuccess;
  if (cols % 8 != 0 || cols > 64 * 8 * 4) return hipErrorInvalidValue;
  if (sl.out && (!sl.row_pos || !sl.page_table || sl.page_size <= 0 || sl.max_pages <= 0))
    return hipErrorInvalidValue;
  const int blocks = (rows + kStatWaves - 1) / kStatWaves + (w1t_rows + kStatWaves - 1) / kStatWaves;
  if (cols <= 64 * 8)
    hipLaunchKernelGGL(row_stats_kernel<1>, dim3(blocks), dim3(64 * kStatWaves), 0, s,
                       static_cast<const uint16_t*>(x), stats, rows, cols, static_cast<const uint16_t*>(w1t),
                       colsum, w1t_rows, sl);
  else
    hipLaunchKernelGGL(row_stats_kernel<4>, dim3(blocks), dim3(64 * kStatWaves), 0, s,
                       static_cast<const uint16_t*>(x), stats, rows, cols, static_cast<const uint16_t*>(w1t),
                       colsum, w1t_rows, sl);
  return hipGetLastError();
}

template <int BM, int BN>
static unsigned gemm_grid(int32_t M, int32_t N) {
  const unsigned tiles = static_cast<unsigned>(((M + BM - 1) / BM) * (N / BN));
  return (tiles + 7u) / 8u * 8u;  // a multiple of the 8 XCDs
}

hipError_t launch_f1_bf16(const void* x, const RowStat* stats, int32_t slots, const float* colsum, const void* w1t,
                          const F1Args& f, int32_t M, int32_t N, int32_t K, hipStream_t s) {
  if (M == 0) return hipSuccess;
  constexpr int BN = 128;
  // a 128-column tile is one head of one chunk
  if (N % BN != 0 || K % GBK != 0 || f.dh != BN || f.inner % BN != 0) return hipErrorInvalidValue;
  if (slots < 1 || slots > kMaxStatSlots || K % slots != 0) return hipErrorInvalidValue;
  if (f.k_pool && !f.row_slots) return hipErrorInvalidValue;
  F1Route r{};
  r.stats = stats;
  r.stat_slots = slots;
  r.eps = f.eps;
  r.row_slots = f.row_slots;
  r.colsum = colsum;
  r.uvqk = static_cast<uint16_t*>(f.uvqk);
  r.inner = f.inner;
  r.kv_to_uvqk = f.kv_to_uvqk;
  r.k_pool = static_cast<uint16_t*>(f.k_pool);
  r.v_pool = static_cast<uint16_t*>(f.v_pool);
  r.pool_layer_offset = f.pool_layer_offset;
  r.dh = f.dh;
  r.page_size = f.page_size;
  r.s_out = static_cast<uint16_t*>(f.s_out);
  // 128-row tiles, or 64-row tiles when the 128-row ones would leave CUs
  // without a second block (few new tokens: candidates over a cached history)
  const auto* A = static_cast<const uint16_t*>(x);
  const auto* B = static_cast<const uint16_t*>(w1t);
#ifndef HSTU_F1_ROW_TILES_AT
#define HSTU_F1_ROW_TILES_AT 512  // 64-row tiles below this many 128-row blocks
#endif
  if ((M + 127) / 128 * (N / BN) < HSTU_F1_ROW_TILES_AT)
    if (K == 8 * GBK)
      hipLaunchKernelGGL((gemm_bf16_kernel<64, BN, 0, 8>), dim3(gemm_grid<64, BN>(M, N)), dim3(256), 0, s, A, B,
                         static_cast<uint16_t*>(f.uvqk), nullptr, r, M, N, K);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<64, BN, 0>), dim3(gemm_grid<64, BN>(M, N)), dim3(256), 0, s, A, B,
                         static_cast<uint16_t*>(f.uvqk), nullptr, r, M, N, K);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<128, BN, 0>), dim3(gemm_grid<128, BN>(M, N)), dim3(256), 0, s, A, B,
                       static_cast<uint16_t*>(f.uvqk), nullptr, r, M, N, K);
  return hipGetLastError();
}

hipError_t launch_head_bf16(const HeadArgs& h, hipStream_t s) {
  if (h.n_rows == 0) return hipSuccess;
  constexpr int BN = kHeadTile;
  const int32_t N = h.tasks * h.hidden;
  if (h.hidden % BN != 0 || h.d % GBK != 0 || h.y_rows <= 0) return hipErrorInvalidValue;
  F1Route r{};
  r.a_rows = h.rows;
  r.a_rows_max = h.y_rows;
  r.h_bias = h.b_hidden;
  r.h_wout = h.w_out;
  r.h_partial = h.partial;
  const auto* y = static_cast<const uint16_t*>(h.y);
  const auto* wt = static_cast<const uint16_t*>(h.w_hidden);
  if (h.n_rows >= 8192)
    hipLaunchKernelGGL((gemm_bf16_kernel<128, BN, 2>), dim3(gemm_grid<128, BN>(h.n_rows, N)), dim3(256), 0, s, y,
                       wt, nullptr, nullptr, r, h.n_rows, N, h.d);
  else
    if (h.d == 8 * GBK)
      hipLaunchKernelGGL((gemm_bf16_kernel<64, BN, 2, 8>), dim3(gemm_grid<64, BN>(h.n_rows, N)), dim3(256), 0, s, y,
                         wt, nullptr, nullptr, r, h.n_rows, N, h.d);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<64, BN, 2>), dim3(gemm_grid<64, BN>(h.n_rows, N)), dim3(256), 0, s, y,
                         wt, nullptr, nullptr, r, h.n_rows, N, h.d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t outs = static_cast<int64_t>(h.n_rows) * h.tasks;
  hipLaunchKernelGGL(head_finalize_kernel, dim3(static_cast<unsigned>((outs + 255) / 256)), dim3(256), 0, s,
                     h.partial, h.hidden / BN, h.tasks, h.b_out, h.logits, h.n_rows);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int epilogue, const void* A, const void* Bm, void* C,
                       const void* R, int32_t M, int32_t N, int32_t K, hipStream_t s, RowStat* y_stats) {
  if (M == 0) return hipSuccess;
  if (dtype == HSTU_BF16) {
    // bf16: f2 (+ residual, epilogue 1) and the backward's plain products
    // (epilogue 3); f1 goes through launch_f1_bf16
    constexpr int BM = 64, BN = 128;
    if ((epilogue != 1 && epilogue != 3) || N % BN != 0 || K % GBK != 0) return hipErrorInvalidValue;
    if (y_stats && epilogue != 1) return hipErrorInvalidValue;
    if (epilogue == 1) {
      F1Route r{};
      r.y_stats = y_stats;
      if (K == 8 * GBK)
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, 1, 8>), dim3(gemm_grid<BM, BN>(M, N)), dim3(256), 0, s,
                           static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bm),
                           static_cast<uint16_t*>(C), static_cast<const uint16_t*>(R), r, M, N, K);
      else
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, 1>), dim3(gemm_grid<BM, BN>(M, N)), dim3(256), 0, s,
                           static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bm),
                           static_cast<uint16_t*>(C), static_cast<const uint16_t*>(R), r, M, N, K);
    } else {
      if (K == 8 * GBK)
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, 3, 8>), dim3(gemm_grid<BM, BN>(M, N)), dim3(256), 0, s,
                           static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bm),
                           static_cast<uint16_t*>(C), nullptr, F1Route{}, M, N, K);
      else
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, 3>), dim3(gemm_grid<BM, BN>(M, N)), dim3(256), 0, s,
                           static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bm),
                           static_cast<uint16_t*>(C), nullptr, F1Route{}, M, N, K);
    }
  } else {
    if (y_stats) return hipErrorInvalidValue;
    dim3 grid((N + FT - 1) / FT, (M + FT - 1) / FT);
    auto a = static_cast<const float*>(A);
    auto b = static_cast<const float*>(Bm);
    auto c = static_cast<float*>(C);
    auto r = static_cast<const float*>(R);
    if (epilogue == 0)
      hipLaunchKernelGGL(gemm_f32_kernel<0>, grid, dim3(256), 0, s, a, b, c, r, M, N, K);
    else
      hipLaunchKernelGGL(gemm_f32_kernel<1>, grid, dim3(256), 0, s, a, b, c, r, M, N, K);
  }
  return hipGetLastError();
}

}  // namespace hstu

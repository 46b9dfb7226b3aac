// Backward of one HSTU layer for training ("How Generative Recommenders Are
// Redefining RecSys at Scale", section HSTU support: HSTU training; the
// forward as in the other kernels: x^ = LayerNorm(x), [U|V|Q|K] = SiLU(x^ W1),
// o = (1/n) sum SiLU(q.k + rab) v, g = LayerNorm(o) * U, y = x + g W2).
// Every position of every user is computed (no cache), keys contiguous.
//
//   gate_bwd_kernel   per row: dU = dg * LN(o), dLN(o) = dg * U through the
//                     LayerNorm to do; also g = LN(o) * U for dW2
//   attn_bwd_kv_kernel  per (user, head, 64 keys): dV and dK of those keys
//                     over every query that sees them, and the rab gradient
//   attn_bwd_q_kernel   per (user, head, 128 queries): dQ over their keys
//   silu_grad_kernel  ds = da * SiLU'(s) (s: the pre-activation of f1)
//   ln_bwd_kernel     per row: dx = LN'(x) applied to dx^, plus dy; also x^
//   wgrad_kernel      weight gradients sum_m A[m][i] B[m][j], split over m
//
// Attention, per visible pair (i, j), with z = q_i.k_j + rab[b(i - j)]:
//   dP = do_i . v_j / n,  dz = dP SiLU'(z),  SiLU'(z) = s(z)(1 + z(1 - s(z))),
//   dv_j += SiLU(z) do_i / n,  dq_i += dz k_j,  dk_j += dz q_i,  drab += dz.
// Both attention kernels recompute z and dP with v_mfma_f32_32x32x16_bf16.
// In the key-block kernel the MFMA rows are queries (read with bits 2 and 3
// of the row swapped, so a lane's score registers hold 8 consecutive queries
// of its key), which makes the score registers the A operand of dV += P^T dO
// and dK += dZ^T Q directly; dO and Q are read transposed from LDS.  The
// query-block kernel is laid out like the forward (rows are keys).
#include <algorithm>

#include "common.h"

namespace hstu {
namespace {

constexpr int DH = 128;
constexpr float kLog2e = 1.44269504088896340736f;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef const __attribute__((address_space(1))) void global_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ void dma16(const uint16_t* src, lds_u16* dst) {
  __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)dst, 16, 0, 0);
}
__device__ __forceinline__ v4i16 lds_read_tr(const lds_u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
// MFMA row i of a 32-row block reads row perm(i): bits 2 and 3 swapped
__device__ __forceinline__ int perm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
// 16-byte-chunk XOR swizzle of [rows][128] bf16 tiles, free of bank
// conflicts for both kinds of operand read: 16 lanes reading one chunk of 16
// consecutive rows see 16 distinct slots (the map is a bijection on row & 15),
// and the transposed reads (4 consecutive rows x 2 adjacent chunks per 16
// lanes) see 8 distinct slots (slot >> 1 differs across the 4 rows).
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ bf16x8 lds_row8(const lds_u16* p) {
  return *(const __attribute__((address_space(3))) bf16x8*)(p);
}
// B-type operand (8 consecutive rows of one column) of a [rows][128] tile
// stored with swz: column block nt (32 columns), rows 16 ks ..
struct TrAddr {
  int a[2][4];
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 5, grp = lane >> 4, j = lane & 15;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 8 * g + 4 * r + (j >> 2);
      const int dcol = 16 * (grp & 1) + 4 * (j & 3);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int d = 32 * nt + dcol;
        a[r][nt] = row * DH + 8 * ((d >> 3) ^ swz(row)) + (d & 7);
      }
    }
  }
  __device__ __forceinline__ bf16x8 read(const lds_u16* t, int nt, int ks) const {
    // whole dwords: extracting the 16-bit elements one by one is lowered
    // incorrectly by this compiler
    u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr(t + a[0][nt] + 16 * ks * DH));
    u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr(t + a[1][nt] + 16 * ks * DH));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
  }
};

__device__ __forceinline__ float sigmoid(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -kLog2e));
}

__device__ __forceinline__ bool visible(int i, int j, int hist) { return j == i || (j < i && j < hist); }

__device__ __forceinline__ void unpack8(u32x4 raw, float* f) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    f[e] = bf2f(static_cast<uint16_t>((e & 1) ? (raw[e >> 1] >> 16) : (raw[e >> 1] & 0xFFFFu)));
}
__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = uint32_t(f2bf(f[2 * k])) | (uint32_t(f2bf(f[2 * k + 1])) << 16);
  return r;
}

// ---------------------------------------------------------------------------
// gate: one wave per row, inner <= 512 (8 values a lane)
// ---------------------------------------------------------------------------
constexpr int kRowsPerBlock = 4;
__global__ __launch_bounds__(64 * kRowsPerBlock) void gate_bwd_kernel(
    const float* __restrict__ o, const uint16_t* __restrict__ a, int64_t a_stride,
    const uint16_t* __restrict__ dg, int32_t rows, int32_t inner, float eps, uint16_t* __restrict__ du,
    uint16_t* __restrict__ dout, uint16_t* __restrict__ g_out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int c0 = 8 * lane;
  const bool on = c0 < inner;
  float ov[8], uv[8], gv[8];
  if (on) {
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(o + static_cast<int64_t>(row) * inner + c0);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(o + static_cast<int64_t>(row) * inner + c0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ov[e] = o0[e];
      ov[4 + e] = o1[e];
    }
    unpack8(*reinterpret_cast<const u32x4*>(a + static_cast<int64_t>(row) * a_stride + c0), uv);
    unpack8(*reinterpret_cast<const u32x4*>(dg + static_cast<int64_t>(row) * inner + c0), gv);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] = uv[e] = gv[e] = 0.f;
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += ov[e];
  const float mean = wave_sum(s) / inner;
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) q += on ? (ov[e] - mean) * (ov[e] - mean) : 0.f;
  const float rstd = 1.0f / sqrtf(wave_sum(q) / inner + eps);
  float lo[8], dln[8], m1 = 0.f, m2 = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = on ? (ov[e] - mean) * rstd : 0.f;
    dln[e] = gv[e] * uv[e];
    m1 += dln[e];
    m2 += dln[e] * lo[e];
  }
  m1 = wave_sum(m1) / inner;
  m2 = wave_sum(m2) / inner;
  if (!on) return;
  float gg[8], dU[8], dO[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    gg[e] = lo[e] * uv[e];
    dU[e] = gv[e] * lo[e];
    dO[e] = rstd * (dln[e] - m1 - lo[e] * m2);
  }
  *reinterpret_cast<u32x4*>(du + static_cast<int64_t>(row) * a_stride + c0) = pack8(dU);
  *reinterpret_cast<u32x4*>(dout + static_cast<int64_t>(row) * inner + c0) = pack8(dO);
  *reinterpret_cast<u32x4*>(g_out + static_cast<int64_t>(row) * inner + c0) = pack8(gg);
}

// ---------------------------------------------------------------------------
// LayerNorm of the input: one wave per row, d <= 2048
// ---------------------------------------------------------------------------
constexpr int kMaxChunks = 4;
__global__ __launch_bounds__(64 * kRowsPerBlock) void ln_bwd_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dxh, const uint16_t* __restrict__ dy,
    int32_t rows, int32_t d, float eps, uint16_t* __restrict__ dx, uint16_t* __restrict__ xhat) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t base = static_cast<int64_t>(row) * d;
  float xv[kMaxChunks][8], gv[kMaxChunks][8];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int col = 8 * (lane + 64 * c);
    if (col < d) {
      unpack8(*reinterpret_cast<const u32x4*>(x + base + col), xv[c]);
      unpack8(*reinterpret_cast<const u32x4*>(dxh + base + col), gv[c]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[c][e] = gv[c][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s += xv[c][e];
  }
  const float mean = wave_sum(s) / d;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) q += (8 * (lane + 64 * c) < d) ? (xv[c][e] - mean) * (xv[c][e] - mean) : 0.f;
  const float rstd = 1.0f / sqrtf(wave_sum(q) / d + eps);
  float m1 = 0.f, m2 = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool on = 8 * (lane + 64 * c) < d;
      xv[c][e] = on ? (xv[c][e] - mean) * rstd : 0.f;  // now x^
      m1 += gv[c][e];
      m2 += gv[c][e] * xv[c][e];
    }
  m1 = wave_sum(m1) / d;
  m2 = wave_sum(m2) / d;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int col = 8 * (lane + 64 * c);
    if (col >= d) continue;
    float yv[8], out[8];
    unpack8(*reinterpret_cast<const u32x4*>(dy + base + col), yv);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = rstd * (gv[c][e] - m1 - xv[c][e] * m2) + yv[e];
    *reinterpret_cast<u32x4*>(dx + base + col) = pack8(out);
    *reinterpret_cast<u32x4*>(xhat + base + col) = pack8(xv[c]);
  }
}

// ds = da * SiLU'(s), 8 values a thread
__global__ __launch_bounds__(256) void silu_grad_kernel(uint16_t* __restrict__ da, const uint16_t* __restrict__ s,
                                                        int64_t n8) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  float dv[8], sv[8];
  unpack8(*reinterpret_cast<const u32x4*>(da + 8 * i), dv);
  unpack8(*reinterpret_cast<const u32x4*>(s + 8 * i), sv);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float sg = sigmoid(sv[e]);
    dv[e] *= sg * (1.0f + sv[e] * (1.0f - sg));
  }
  *reinterpret_cast<u32x4*>(da + 8 * i) = pack8(dv);
}

// ---------------------------------------------------------------------------
// weight gradients: part[split][i][j] = sum over the split's m of A[m][i] B[m][j]
// 128 x 128 tiles, 4 waves as 2 x 2, m in steps of 64 through double-buffered
// LDS tiles [64 m][128] filled by direct copies; both operands are read
// transposed (8 consecutive m of one column).  Rows past the split's end copy
// from a row of zeros.
// ---------------------------------------------------------------------------
constexpr int WT = 128, WK = 64;
__global__ __launch_bounds__(256, 2) void wgrad_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                       const uint16_t* __restrict__ B, int64_t ldb, int32_t M,
                                                       int32_t N1, int32_t N2, int32_t m_chunk,
                                                       const uint16_t* __restrict__ zeros,
                                                       float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t A0s[WK * WT];
  __shared__ __attribute__((aligned(16))) uint16_t A1s[WK * WT];
  __shared__ __attribute__((aligned(16))) uint16_t B0s[WK * WT];
  __shared__ __attribute__((aligned(16))) uint16_t B1s[WK * WT];
  lds_u16* const A0 = (lds_u16*)A0s;
  lds_u16* const A1 = (lds_u16*)A1s;
  lds_u16* const B0 = (lds_u16*)B0s;
  lds_u16* const B1 = (lds_u16*)B1s;
  const int tn2 = N2 / WT;
  const int tiles = (N1 / WT) * tn2;
  const int split = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int i0 = (tile / tn2) * WT, j0 = (tile % tn2) * WT;
  const int m_begin = split * m_chunk, m_end = min(M, m_begin + m_chunk);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = uniform(tid >> 6), wm = wave >> 1, wn = wave & 1;
  const int lrow = lane >> 4, lslot = lane & 15;
  auto copy = [&](int m0, lds_u16* Ad, lds_u16* Bd) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * i + lrow;
      const int m = m0 + r;
      const int ch = 8 * (lslot ^ swz(r));
      const uint16_t* sa = m < m_end ? A + static_cast<int64_t>(m) * lda + i0 + ch : zeros + ch;
      const uint16_t* sb = m < m_end ? B + static_cast<int64_t>(m) * ldb + j0 + ch : zeros + ch;
      dma16(sa, Ad + (16 * wave + 4 * i) * WT);
      dma16(sb, Bd + (16 * wave + 4 * i) * WT);
    }
  };
  TrAddr tr;
  tr.init(lane);
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  auto mma = [&](const lds_u16* As, const lds_u16* Bs) {
#pragma unroll
    for (int ks = 0; ks < WK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = tr.read(As, 2 * wm + i, ks);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = tr.read(Bs, 2 * wn + j, ks);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };
  const int steps = (m_end - m_begin + WK - 1) / WK;
  if (steps > 0) copy(m_begin, A0, B0);
  __syncthreads();
  for (int st = 0; st < steps; st += 2) {
    if (st + 1 < steps) copy(m_begin + (st + 1) * WK, A1, B1);
    __builtin_amdgcn_sched_barrier(0);
    mma(A0, B0);
    __syncthreads();
    if (st + 1 >= steps) break;
    if (st + 2 < steps) copy(m_begin + (st + 2) * WK, A0, B0);
    __builtin_amdgcn_sched_barrier(0);
    mma(A1, B1);
    __syncthreads();
  }
  // C rows i (first operand), columns j: lane holds column l32 of each block
  float* out = part + static_cast<int64_t>(split) * N1 * N2;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + 32 * (2 * wm + i) + 8 * (r >> 2) + 4 * g + (r & 3);
        const int col = j0 + 32 * (2 * wn + j) + l32;
        out[static_cast<int64_t>(row) * N2 + col] = acc[i][j][r];
      }
}

// out[e] = sum over s of part[s][e], in split order
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, int32_t splits, int64_t n,
                                                        float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int k = 0; k < splits; ++k) s += part[static_cast<int64_t>(k) * n + i];
  out[i] = s;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint16_t* __restrict__ p, int32_t n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------------------
// attention, per 64-key block: dK, dV and the rab gradient
// ---------------------------------------------------------------------------
// Two key groups of 32, each taken by two waves with split roles, so that
// each pair's S and dP are computed once and a wave fits in half the
// register file (two blocks share a CU); the block's K and V rows sit in
// LDS.  A step covers 32 queries.  Wave A of a group computes z = S + bias,
// passes it to wave B through the group's LDS scratch, and accumulates dV
// over all head dims; wave B computes dP, forms dz from it and z, sums the
// rab gradient and accumulates dK over all head dims.  The rab gradient is
// summed per distance i - j in LDS (wave B gathers its 32 x 32 pairs by
// distance across lanes and adds one sum per distance; when its pairs fall
// in at most four buckets it adds one wave sum per bucket), distances past
// the LDS window (ragged tail steps) straight into their bucket; the sums
// are folded into buckets and written as this item's partial.
constexpr int KB = kBwdKeyBlock;  // keys per item: 2 groups of 32, each split over two waves by head dims
constexpr int QT = 32;            // queries per step
constexpr int kTab = QT + KB;     // distances per step (95 used)
constexpr int kDistWin = 256;     // distances summed in LDS; larger ones (ragged tail steps) go to their bucket

__global__ __launch_bounds__(256, 2) void attn_bwd_kv_kernel(BwdLaunch b) {
  __shared__ __attribute__((aligned(16))) uint16_t Q0s[QT * DH];
  __shared__ __attribute__((aligned(16))) uint16_t D0s[QT * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Q1s[QT * DH];
  __shared__ __attribute__((aligned(16))) uint16_t D1s[QT * DH];
  __shared__ float bias0[kTab], bias1[kTab];
  // rab-gradient sums, private to each key group's summing wave (one writer
  // each, adds in program order: the result does not depend on scheduling)
  __shared__ float drab_s[2][256];      // per bucket
  __shared__ float dist_s[2][kDistWin];  // per distance
  __shared__ float far_s[2][64];         // a step's sums at distances past the window, per lane
  __shared__ float diag_s[2 * 32 * 33];  // per-key-group scratch of the distance sums
  __shared__ __attribute__((aligned(16))) uint16_t Kts[KB * DH];  // the block's keys: K and V rows
  __shared__ __attribute__((aligned(16))) uint16_t Vts[KB * DH];
  lds_u16* const Q0 = (lds_u16*)Q0s;
  lds_u16* const D0 = (lds_u16*)D0s;
  lds_u16* const Q1 = (lds_u16*)Q1s;
  lds_u16* const D1 = (lds_u16*)D1s;

  const BwdKVItem it = b.kv_items[blockIdx.x];
  const UserInfo us = b.plan.users[it.user];
  const int h = it.head, k0 = it.k0;
  const int L = us.kv_len, hist = us.hist, row0 = us.q_row0;
  const float inv_n = us.inv_n;
  const int nb = b.num_buckets;
  const int inner = b.plan.H * DH;
  const int64_t ST = 4 * static_cast<int64_t>(inner);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = uniform(tid >> 6);
  const int kg = wave >> 1;                 // key group
  const bool role_b = (wave & 1) != 0;      // A: z and dV; B: dP, dz, the rab gradient and dK
  const int kw0 = k0 + 32 * kg;
  const int key = kw0 + l32;
  const int ndist = L - k0;  // distances 0 .. L - 1 - k0 can occur
  for (int i = tid; i < 2 * 256; i += 256) drab_s[i >> 8][i & 255] = 0.f;
  for (int i = tid; i < 2 * kDistWin; i += 256) dist_s[i / kDistWin][i % kDistWin] = 0.f;
  lds_u16* const Kt = (lds_u16*)Kts;
  lds_u16* const Vt = (lds_u16*)Vts;
  const int lrow = lane >> 4, lslot = lane & 15;
  // the block's K and V rows, staged once (wave w fills rows 16 w .. 16 w + 15);
  // they are the B operands of S = Q K^T and dP = dO V^T
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * wave + 4 * i + lrow;
    const int kc = min(k0 + r, L - 1);
    const int ch = 8 * (lslot ^ swz(r));
    const uint16_t* src = b.a + (row0 + kc) * ST + h * DH + ch;
    dma16(src + 3 * inner, Kt + (16 * wave + 4 * i) * DH);
    dma16(src + 1 * inner, Vt + (16 * wave + 4 * i) * DH);
  }
  // dV (wave A) or dK (wave B) of this group's 32 keys over all head dims
  f32x16 gacc[DH / 32];
#pragma unroll
  for (int t = 0; t < DH / 32; ++t) gacc[t] = f32x16{};

  // query steps that see some key of the block
  const int kb_end = min(k0 + KB, L);
  auto step_vis = [&](int q0) {
    const int qe = min(q0 + QT, L);
    if (k0 < qe && q0 < kb_end) return true;
    return k0 < hist && k0 < qe - 1;
  };
  // copy: wave w fills rows 8 w .. 8 w + 7 of Q and dO, four rows per instruction
  auto copy_tile = [&](int q0, lds_u16* Qd, lds_u16* Dd) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * wave + 4 * i + lrow;
      const int q = min(q0 + r, L - 1);
      const int ch = 8 * (lslot ^ swz(r));
      dma16(b.a + (row0 + q) * ST + 2 * inner + h * DH + ch, Qd + (8 * wave + 4 * i) * DH);
      dma16(b.dO + static_cast<int64_t>(row0 + q) * inner + h * DH + ch, Dd + (8 * wave + 4 * i) * DH);
    }
  };
  // distance table of a step: entry t is distance (q0 - k0 - (KB - 1)) + t
  auto fill_tab = [&](int q0, float* bias) {
    if (tid < kTab) {
      const int d = q0 - k0 - (KB - 1) + tid;
      bias[tid] = d < 0 ? 0.f : b.rab[rel_bucket(d, nb)];
    }
  };
  // transposed-read addresses of the four column blocks
  TrAddr tr;
  tr.init(lane);
  // A operand of S: query row perm(l32); B operand: this lane's key row
  // 32 kg + l32; chunk (2s + g) of each, swizzled (formed per use to save registers)
  const int qrow = perm(l32), krow = 32 * kg + l32;
  const int qbase = qrow * DH, qx = swz(qrow), kbase = krow * DH, kx = swz(krow);

  // Per-distance sums of a half's dz (register r of lane (l, g) holds key
  // offset l and query offset 16 (r / 8) + 8 g + r % 8, at distance D + that
  // offset - l, D = qh - kw0): the wave writes its 32 x 32 tile to its own
  // LDS scratch, each lane sums one diagonal (query offset - key offset =
  // lane - 31) and adds it to its distance's sum (the lanes' distances are
  // distinct, so one plain add each).  Distances past the window (ragged
  // tail steps) go to their buckets one lane after another.  Float LDS
  // atomics are slow on this chip (one per pair cost more than the rest of
  // the step) and would make the sums depend on scheduling.  The scratch is
  // private to the wave and a wave's LDS operations complete in order, so no
  // barrier is needed between the writes and the reads.
  float* const scr = diag_s + kg * (32 * 33);
  auto diag_add = [&](int qh, const f32x16& dz) {
#pragma unroll
    for (int r = 0; r < 16; ++r) scr[(16 * (r >> 3) + 8 * g + (r & 7)) * 33 + l32] = dz[r];
    const int e = lane - 31;
    float acc = 0.f;
#pragma unroll 8
    for (int t = 0; t < 32; ++t) {
      const int qo = t + e;
      acc += (qo >= 0 && qo < 32) ? scr[min(max(qo, 0), 31) * 33 + t] : 0.f;
    }
    const int d = qh - kw0 + e;
    const bool in = d >= 0 && d < ndist;
    if (in && d < kDistWin) dist_s[kg][d] += acc;
    if (__any(in && d >= kDistWin)) {
      far_s[kg][lane] = in && d >= kDistWin ? acc : 0.f;
      if (lane == 0) {
        for (int l = 0; l < 64; ++l) {
          const int dl = qh - kw0 + l - 31;
          if (dl >= kDistWin && dl < ndist) drab_s[kg][rel_bucket(dl, nb)] += far_s[kg][l];
        }
      }
    }
  };
  // register r holds query q0 + 16 (r / 8) + 8 g + r % 8 against this lane's
  // key, and z[r] the pair's q.k + rab.  Masked pairs count zero.
  auto visible = [&](int qh, int r) {
    const int i = qh + 16 * (r >> 3) + 8 * g + (r & 7);
    return (i < L) & (key < L) & ((key == i) | ((key < i) & (key < hist)));
  };
  auto full_step = [&](int qh) { return kw0 + 31 < qh && kw0 + 31 < hist && qh + 32 <= L && kw0 + 31 < L; };
  // wave A: z into the A operands' weights p = SiLU(z) / n
  auto weights_p = [&](int qh, f32x16& z) {
    if (full_step(qh)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = z[r] * sigmoid(z[r]) * inv_n;
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = visible(qh, r) ? z[r] * sigmoid(z[r]) * inv_n : 0.f;
    }
  };
  // wave B: dP into dz = dP / n * SiLU'(z), and the rab gradient.  Wave-uniform
  // cases, each a straight loop: every pair visible in one bucket (one wave
  // sum) or in at most four (one wave sum per bucket, split at the bucket
  // edges), every pair visible (sums per distance), or masked (sums per
  // distance).
  auto gradient_dz = [&](int qh, const f32x16& z, f32x16& pacc) {
    const int dmin = qh - (kw0 + 31), dmax = qh + 31 - kw0;
    const bool full = full_step(qh);
    const bool uni = full && rel_bucket(dmin, nb) == rel_bucket(dmax, nb);
    const int sb = qh - key;  // distance of register 0
    auto dz_of = [&](int r) {
      const float sg = sigmoid(z[r]);
      return pacc[r] * inv_n * sg * (1.0f + z[r] * (1.0f - sg));
    };
    // up to four buckets: t[k] is the first distance of bucket blo + 1 + k
    const int blo = full ? rel_bucket(dmin, nb) : 0;
    const int bhi = full ? rel_bucket(dmax, nb) : 0;
    const bool few = full && bhi - blo <= 3;
    if (uni) {
      float dsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pacc[r] = dz_of(r);
        dsum += pacc[r];
      }
      dsum = wave_sum(dsum);
      if (lane == 0) drab_s[kg][bhi] += dsum;
    } else if (few) {
      int t[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        if (blo + 1 + k > bhi) {
          t[k] = 1 << 30;
          continue;
        }
        int lo = dmin, hi = dmax;  // bucket(lo) < blo + 1 + k <= bucket(hi)
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (rel_bucket(mid, nb) >= blo + 1 + k) hi = mid; else lo = mid;
        }
        t[k] = hi;
      }
      float s_all = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dz = dz_of(r);
        pacc[r] = dz;
        const int dd = sb + 16 * (r >> 3) + 8 * g + (r & 7);
        s_all += dz;
        s1 += dd >= t[0] ? dz : 0.f;
        s2 += dd >= t[1] ? dz : 0.f;
        s3 += dd >= t[2] ? dz : 0.f;
      }
      s_all = wave_sum(s_all);
      s1 = wave_sum(s1);
      s2 = wave_sum(s2);
      s3 = wave_sum(s3);
      if (lane == 0) {
        drab_s[kg][blo] += s_all - s1;
        if (blo + 1 <= bhi) drab_s[kg][blo + 1] += s1 - s2;
        if (blo + 2 <= bhi) drab_s[kg][blo + 2] += s2 - s3;
        if (blo + 3 <= bhi) drab_s[kg][blo + 3] += s3;
      }
    } else if (full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) pacc[r] = dz_of(r);
      diag_add(qh, pacc);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) pacc[r] = visible(qh, r) ? dz_of(r) : 0.f;
      diag_add(qh, pacc);
    }
  };
  // wave A: dV += P^T dO; wave B: dK += dZ^T Q, over the step's 32 queries
  // and all head dims
  auto accumulate = [&](const f32x16& w, const lds_u16* T) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 wa;
#pragma unroll
      for (int e = 0; e < 8; ++e) wa[e] = static_cast<__bf16>(w[8 * ks + e]);
#pragma unroll
      for (int t = 0; t < DH / 32; ++t)
        gacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, tr.read(T, t, ks), gacc[t], 0, 0, 0);
    }
  };
  // z (wave A) or dP (wave B) over all head dims; z passes through the key
  // group's scratch, in the layout the distance sums use (wave B reads it
  // before its own sums overwrite it; wave A writes the next step's after
  // the step's closing barrier).  Every wave reaches the barrier in between.
  auto step = [&](int q0, const lds_u16* Qs, const lds_u16* Ds, const float* bias) {
    const bool active = kw0 < L;
    f32x16 acc = f32x16{};
    if (active) {
      const lds_u16* Xs = role_b ? Ds : Qs;
      const lds_u16* Ys = role_b ? Vt : Kt;
#pragma unroll
      for (int s = 0; s < DH / 16; ++s) {
        const int qa_s = qbase + 8 * ((2 * s + g) ^ qx), ka_s = kbase + 8 * ((2 * s + g) ^ kx);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(Xs + qa_s), lds_row8(Ys + ka_s), acc, 0, 0, 0);
      }
      if (!role_b) {
        const int tb = (KB - 1) - (key - k0);  // table entry of register 0
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc[r] += bias[tb + 16 * (r >> 3) + 8 * g + (r & 7)];
          scr[(16 * (r >> 3) + 8 * g + (r & 7)) * 33 + l32] = acc[r];
        }
      }
    }
    __syncthreads();  // z of the step in the scratch
    if (active) {
      if (!role_b) {
        weights_p(q0, acc);
        accumulate(acc, Ds);
      } else {
        f32x16 z;
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = scr[(16 * (r >> 3) + 8 * g + (r & 7)) * 33 + l32];
        gradient_dz(q0, z, acc);
        accumulate(acc, Qs);
      }
    }
  };

  int q0 = (k0 / QT) * QT;
  while (q0 < L && !step_vis(q0)) q0 += QT;
  if (q0 < L) {
    fill_tab(q0, bias0);
    copy_tile(q0, Q0, D0);
  }
  __syncthreads();  // tables zeroed, first step staged
  while (q0 < L) {
    int qn = q0 + QT;
    while (qn < L && !step_vis(qn)) qn += QT;
    if (qn < L) {
      fill_tab(qn, bias1);
      copy_tile(qn, Q1, D1);
    }
    __builtin_amdgcn_sched_barrier(0);
    step(q0, Q0, D0, bias0);
    __syncthreads();
    if (qn >= L) break;
    q0 = qn;
    qn = q0 + QT;
    while (qn < L && !step_vis(qn)) qn += QT;
    if (qn < L) {
      fill_tab(qn, bias0);
      copy_tile(qn, Q0, D0);
    }
    __builtin_amdgcn_sched_barrier(0);
    step(q0, Q1, D1, bias1);
    __syncthreads();
    q0 = qn;
  }
  __syncthreads();
  // this item's partial, one bucket a thread, in a fixed order: the two key
  // groups' bucket sums, then their per-distance sums in increasing distance
  // (buckets grow with distance, so bucket k's distances are one range,
  // found by bisection)
  const int dend = min(ndist, kDistWin);
  auto first_at_least = [&](int kk) {  // first distance in [0, dend) of bucket >= kk, or dend
    int lo = 0, hi = dend;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (rel_bucket(mid, nb) >= kk) hi = mid; else lo = mid + 1;
    }
    return lo;
  };
  for (int k = tid; k < nb; k += 256) {
    float sum = drab_s[0][k] + drab_s[1][k];
    const int d1 = first_at_least(k + 1);
    for (int d = first_at_least(k); d < d1; ++d) sum += dist_s[0][d] + dist_s[1][d];
    b.drab_partial[static_cast<int64_t>(blockIdx.x) * nb + k] = sum;
  }
  // rows (keys) 8 (r / 4) + 4 g + r % 4 of this group's 32, column 32 t + l32:
  // dV (chunk 1 of da) from wave A, dK (chunk 3) from wave B
#pragma unroll
  for (int t = 0; t < DH / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = kw0 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (kk < L)
        b.da[(row0 + kk) * ST + (role_b ? 3 : 1) * inner + h * DH + 32 * t + l32] = f2bf(gacc[t][r]);
    }
}

// ---------------------------------------------------------------------------
// attention, per 128-query block: dQ
// ---------------------------------------------------------------------------
constexpr int KT = 64;  // keys per step

__global__ __launch_bounds__(256, 1) void attn_bwd_q_kernel(BwdLaunch b) {
  __shared__ __attribute__((aligned(16))) uint16_t K0s[KT * DH];
  __shared__ __attribute__((aligned(16))) uint16_t V0s[KT * DH];
  __shared__ __attribute__((aligned(16))) uint16_t K1s[KT * DH];
  __shared__ __attribute__((aligned(16))) uint16_t V1s[KT * DH];
  __shared__ float bias0[256], bias1[256];
  lds_u16* const K0 = (lds_u16*)K0s;
  lds_u16* const V0 = (lds_u16*)V0s;
  lds_u16* const K1 = (lds_u16*)K1s;
  lds_u16* const V1 = (lds_u16*)V1s;

  const BwdQItem it = b.q_items[blockIdx.x];
  const QBlock qb = b.plan.qblocks[it.qblock];
  const UserInfo us = b.plan.users[qb.user];
  const int h = it.head;
  const int L = us.kv_len, hist = us.hist, row0 = us.q_row0;
  const float inv_n = us.inv_n;
  const int nb = b.num_buckets;
  const int inner = b.plan.H * DH;
  const int64_t ST = 4 * static_cast<int64_t>(inner);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = uniform(tid >> 6);
  const int wq0 = 32 * wave;
  const bool wave_active = wq0 < qb.count;
  const int qlocal = wq0 + l32;
  const int qpos = qb.pos0 + qlocal;
  const int qa = qb.pos0, qe = qb.pos0 + qb.count;
  // Q and dO of this lane's query as B operands (S^T = K Q^T, dP^T = V dO^T)
  bf16x8 qf[DH / 16], df[DH / 16];
  {
    const int qc = min(qlocal, qb.count - 1);
    const uint16_t* qr = b.a + (qb.row0 + qc) * ST + 2 * inner + h * DH;
    const uint16_t* dr = b.dO + static_cast<int64_t>(qb.row0 + qc) * inner + h * DH;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qr + 16 * s + 8 * g));
      df[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dr + 16 * s + 8 * g));
    }
  }
  f32x16 dq_acc[DH / 32];
#pragma unroll
  for (int t = 0; t < DH / 32; ++t) dq_acc[t] = f32x16{};

  auto tile_vis = [&](int k0) {
    if (k0 < qe && qa < k0 + KT) return true;
    return k0 < hist && k0 < qe - 1;
  };
  const int lrow = lane >> 4, lslot = lane & 15;
  auto copy_tile = [&](int k0, lds_u16* Kd, lds_u16* Vd) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * i + lrow;
      const int kk = min(k0 + r, L - 1);
      const uint16_t* src = b.a + (row0 + kk) * ST + h * DH;
      dma16(src + 3 * inner + 8 * (lslot ^ swz(r)), Kd + (16 * wave + 4 * i) * DH);
      dma16(src + 1 * inner + 8 * (lslot ^ swz(r)), Vd + (16 * wave + 4 * i) * DH);
    }
  };
  // reversed distance table: entry t is distance qa + 127 - k0 - t
  auto fill_bias = [&](int k0, float* bias) {
    if (tid < 128 + KT - 1) {
      const int d = qa + 127 - k0 - tid;
      bias[tid] = d < 0 ? 0.f : b.rab[rel_bucket(d, nb)];
    }
  };
  TrAddr tr;
  tr.init(lane);
  int kaddr[DH / 16], vaddr[DH / 16];  // A operands: key row perm(l32), chunk (2 s + g)
  {
    const int row = perm(l32);
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      kaddr[s] = row * DH + 8 * ((2 * s + g) ^ swz(row));
      vaddr[s] = row * DH + 8 * ((2 * s + g) ^ swz(row));
    }
  }

  auto step = [&](int k0, const lds_u16* Ks, const lds_u16* Vs, const float* bias) {
    f32x16 sacc[KT / 32], pacc[KT / 32];
#pragma unroll
    for (int mt = 0; mt < KT / 32; ++mt) {
      sacc[mt] = pacc[mt] = f32x16{};
#pragma unroll
      for (int s = 0; s < DH / 16; ++s) {
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(Ks + kaddr[s] + 32 * mt * DH), qf[s], sacc[mt], 0, 0, 0);
        pacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(Vs + vaddr[s] + 32 * mt * DH), df[s], pacc[mt], 0, 0, 0);
      }
    }
    // register r of block mt: key k0 + 32 mt + 16 (r / 8) + 8 g + r % 8, query qpos;
    // no mask when every key of the step is visible to every query of the wave
    const float* brow = &bias[127 - qlocal + 8 * g];
    const bool full = k0 + KT - 1 < qa + wq0 && k0 + KT - 1 < hist && k0 + KT <= L && wq0 + 32 <= qb.count;
    if (full) {
#pragma unroll
      for (int mt = 0; mt < KT / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int koff = 32 * mt + 16 * (r >> 3) + (r & 7);
          const float z = sacc[mt][r] + brow[koff];
          const float sg = sigmoid(z);
          sacc[mt][r] = pacc[mt][r] * inv_n * sg * (1.0f + z * (1.0f - sg));
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < KT / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int koff = 32 * mt + 16 * (r >> 3) + (r & 7);
          const int j = k0 + 8 * g + koff;
          const float z = sacc[mt][r] + brow[koff];
          const float sg = sigmoid(z);
          const float dz = pacc[mt][r] * inv_n * sg * (1.0f + z * (1.0f - sg));
          const bool vis = (j < L) & (qlocal < qb.count) & ((j == qpos) | ((j < qpos) & (j < hist)));
          sacc[mt][r] = vis ? dz : 0.f;
        }
    }
    // dQ += dZ K (k = the step's keys; K read transposed)
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      bf16x8 za;
#pragma unroll
      for (int e = 0; e < 8; ++e) za[e] = static_cast<__bf16>(sacc[ks >> 1][8 * (ks & 1) + e]);
#pragma unroll
      for (int nt = 0; nt < DH / 32; ++nt)
        dq_acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(za, tr.read(Ks, nt, ks), dq_acc[nt], 0, 0, 0);
    }
  };

  int k0 = 0;
  while (k0 < L && !tile_vis(k0)) k0 += KT;
  if (k0 < L) {
    fill_bias(k0, bias0);
    copy_tile(k0, K0, V0);
  }
  __syncthreads();
  while (k0 < L) {
    int kn = k0 + KT;
    while (kn < L && !tile_vis(kn)) kn += KT;
    if (kn < L) {
      fill_bias(kn, bias1);
      copy_tile(kn, K1, V1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (wave_active) step(k0, K0, V0, bias0);
    __syncthreads();
    if (kn >= L) break;
    k0 = kn;
    kn = k0 + KT;
    while (kn < L && !tile_vis(kn)) kn += KT;
    if (kn < L) {
      fill_bias(kn, bias0);
      copy_tile(kn, K0, V0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (wave_active) step(k0, K1, V1, bias1);
    __syncthreads();
    k0 = kn;
  }
  if (!wave_active) return;
  // rows (queries) wq0 + 8 (r / 4) + 4 g + r % 4, column 32 nt + l32
#pragma unroll
  for (int nt = 0; nt < DH / 32; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ql = wq0 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (ql < qb.count)
        b.da[(qb.row0 + ql) * ST + 2 * inner + h * DH + 32 * nt + l32] = f2bf(dq_acc[nt][r]);
    }
}

}  // namespace

hipError_t launch_gate_bwd(const float* o, const void* a, int64_t a_stride, const void* dg, int32_t rows,
                           int32_t inner, float eps, void* du, void* dout, void* g, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (inner > 512 || inner % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gate_bwd_kernel, dim3((rows + kRowsPerBlock - 1) / kRowsPerBlock), dim3(64 * kRowsPerBlock), 0,
                     s, o, static_cast<const uint16_t*>(a), a_stride, static_cast<const uint16_t*>(dg), rows, inner,
                     eps, static_cast<uint16_t*>(du), static_cast<uint16_t*>(dout), static_cast<uint16_t*>(g));
  return hipGetLastError();
}

hipError_t launch_ln_bwd(const void* x, const void* dxh, const void* dy, int32_t rows, int32_t d, float eps, void* dx,
                         void* xhat, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (d % 8 || d > 64 * 8 * kMaxChunks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ln_bwd_kernel, dim3((rows + kRowsPerBlock - 1) / kRowsPerBlock), dim3(64 * kRowsPerBlock), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(dxh),
                     static_cast<const uint16_t*>(dy), rows, d, eps, static_cast<uint16_t*>(dx),
                     static_cast<uint16_t*>(xhat));
  return hipGetLastError();
}

hipError_t launch_silu_grad(void* da, const void* s_pre, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(silu_grad_kernel, dim3(static_cast<unsigned>((n8 + 255) / 256)), dim3(256), 0, s,
                     static_cast<uint16_t*>(da), static_cast<const uint16_t*>(s_pre), n8);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, int32_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, static_cast<uint16_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_wgrad(const void* A, int64_t lda, const void* B, int64_t ldb, int32_t M, int32_t N1, int32_t N2,
                        int32_t splits, const void* zeros, float* part, float* out, hipStream_t s) {
  if (N1 % WT || N2 % WT || splits < 1) return hipErrorInvalidValue;
  const int64_t n = static_cast<int64_t>(N1) * N2;
  if (M == 0) {  // no rows: zero gradients (a sum over no splits)
    hipLaunchKernelGGL(split_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, part, 0, n,
                       out);
    return hipGetLastError();
  }
  int32_t chunk = (M + splits - 1) / splits;
  chunk = (chunk + WK - 1) / WK * WK;
  const int32_t used = (M + chunk - 1) / chunk;
  const unsigned blocks = static_cast<unsigned>((N1 / WT) * (N2 / WT) * used);
  hipLaunchKernelGGL(wgrad_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint16_t*>(A), lda,
                     static_cast<const uint16_t*>(B), ldb, M, N1, N2, chunk, static_cast<const uint16_t*>(zeros),
                     part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(split_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, part, used, n,
                     out);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const BwdLaunch& b, hipStream_t s) {
  if (b.n_kv_items > 0)
    hipLaunchKernelGGL(attn_bwd_kv_kernel, dim3(static_cast<unsigned>(b.n_kv_items)), dim3(256), 0, s, b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (b.n_q_items > 0)
    hipLaunchKernelGGL(attn_bwd_q_kernel, dim3(static_cast<unsigned>(b.n_q_items)), dim3(256), 0, s, b);
  return hipGetLastError();
}

// drab[k] = sum over items of partial[item][k]: one block per bucket, thread
// t sums items t, t + 256, ... in order, then a fixed-order tree
namespace {
__global__ __launch_bounds__(256) void drab_sum_kernel(const float* __restrict__ part, int32_t items, int32_t nb,
                                                       float* __restrict__ drab) {
  __shared__ float red[256];
  const int k = blockIdx.x, t = threadIdx.x;
  float s = 0.f;
  for (int i = t; i < items; i += 256) s += part[static_cast<int64_t>(i) * nb + k];
  red[t] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) drab[k] = red[0];
}
}  // namespace

hipError_t launch_drab_sum(const float* part, int32_t items, int32_t nb, float* drab, hipStream_t s) {
  hipLaunchKernelGGL(drab_sum_kernel, dim3(nb), dim3(256), 0, s, part, items, nb, drab);
  return hipGetLastError();
}

}  // namespace hstu

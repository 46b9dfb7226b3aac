// The two projections of the HSTU layer ("How Generative Recommenders Are
// Redefining RecSys at Scale", section HSTU):
//   f1: [U|V|Q|K] = SiLU(LayerNorm(x) . W1)   (epilogue 0)
//   f2: y = x + g . W2                        (epilogue 1)
// Matrices are row-major: A [M][K], B [K][N] (the weight layout), C [M][N].
//
// bf16 kernel: a BM x 128 output tile per 256-thread block (4 waves as 2 x 2,
// each wave (BM/2) x 64 as v_mfma_f32_32x32x16_bf16 tiles), K staged 64 at a
// time through LDS.  Each MFMA multiplies a W^T fragment by an x^T fragment,
// producing C^T tiles, so a lane owns 4 consecutive output columns of one row
// and stores (and reads the residual) 8 bytes at a time.  B tiles are written
// to LDS transposed (n-major) because the MFMA wants 8 consecutive k per lane;
// both LDS tiles use a 16-byte-chunk XOR swizzle so the transposing writes and
// the operand reads are free of bank conflicts.  The next K tile is fetched
// into registers while the current one is multiplied.
//
// Epilogue 0 applies the pre-norm algebraically: with mu, rstd the row
// statistics of x and s_n = sum_k W1[k][n],
//     LayerNorm(x) . W1 = rstd * (x . W1 - mu * s_n),
// so x is multiplied as stored (no normalised copy) and s_n is accumulated
// while W1 is staged.  The SiLU'd columns are routed by chunk: U and Q to the
// token-major buffer, K and V either to the same buffer (contiguous keys) or
// straight into their pages (paged cache; the append of the new tokens).
//
// fp32: plain 64 x 64-tile FMA kernels, with the pre-norm done by a separate
// row LayerNorm and the append by the copy kernel.
#include "common.h"

namespace hstu {
namespace {

constexpr int GBN = 128, GBK = 64;

__device__ __forceinline__ float epi_silu(float x) { return x / (1.0f + __expf(-x)); }

__device__ __forceinline__ int swz_a(int m, int c) { return c ^ (m & 7); }
__device__ __forceinline__ int swz_b(int n, int c) { return c ^ ((n + (n >> 3)) & 7); }

// Routing of f1's output columns (epilogue 0).
struct F1Route {
  const float2* stats;       // [M] (mean, rstd) of the input rows
  uint16_t* uvqk;            // [M][4 inner] token-major destination
  int32_t inner;             // H * dh
  bool kv_to_uvqk;           // also write the K and V chunks to uvqk
  // paged K/V destination (k_pool == nullptr: none)
  uint16_t* k_pool;
  uint16_t* v_pool;
  int64_t pool_layer_offset;  // elements
  const int32_t* page_table;  // [B][max_pages]
  const int32_t* new_offsets; // [B+1]
  const int32_t* start_pos;   // [B]
  int32_t B, max_pages, num_pages, H, dh, page_size;
};

template <int BM, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ Bm,
                                                           uint16_t* __restrict__ C,
                                                           const uint16_t* __restrict__ R,
                                                           F1Route route, int32_t M, int32_t N,
                                                           int32_t K) {
  constexpr int MT = BM / 64;  // 32-row MFMA tiles per wave along m
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * GBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bt[GBN * GBK];
  __shared__ float colsum_part[EPI == 0 ? 16 * GBN : 1];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_tiles_n = N / GBN;
  const int m0 = (blockIdx.x / n_tiles_n) * BM;
  const int n0 = (blockIdx.x % n_tiles_n) * GBN;

  // global -> register staging: A: rows tid/8 + 32 i, chunk tid%8;
  // B: 2 rounds x 2 rows (k pair 2*(tid/16) + 32 r), n chunk tid%16
  u32x4 ra[BM / 32], rb[4];
  float csum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
      int m = m0 + tid / 8 + 32 * i;
      int c = tid % 8;
      ra[i] = m < M ? *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(m) * K + k0 + 8 * c)
                    : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      int k = k0 + 2 * (tid / 16) + 32 * r;
      int n = n0 + 8 * (tid % 16);
      rb[2 * r] = *reinterpret_cast<const u32x4*>(Bm + static_cast<int64_t>(k) * N + n);
      rb[2 * r + 1] = *reinterpret_cast<const u32x4*>(Bm + static_cast<int64_t>(k + 1) * N + n);
    }
  };
  auto store_tiles = [&]() {
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
      int m = tid / 8 + 32 * i, c = tid % 8;
      *reinterpret_cast<u32x4*>(&As[m * GBK + 8 * swz_a(m, c)]) = ra[i];
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      int kk = 2 * (tid / 16) + 32 * r;  // even k within the tile
      int nb = 8 * (tid % 16);
      u32x4 lo = rb[2 * r], hi = rb[2 * r + 1];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t a = (j & 1) ? (lo[j >> 1] >> 16) : (lo[j >> 1] & 0xFFFFu);
        uint32_t b = (j & 1) ? (hi[j >> 1] >> 16) : (hi[j >> 1] & 0xFFFFu);
        if (EPI == 0) csum[j] += bf2f(static_cast<uint16_t>(a)) + bf2f(static_cast<uint16_t>(b));
        int n = nb + j;
        int chunk = swz_b(n, kk >> 3);
        *reinterpret_cast<uint32_t*>(&Bt[n * GBK + 8 * chunk + (kk & 7)]) = a | (b << 16);
      }
    }
  };

  f32x16 acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = K / GBK;
  load_tiles(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    store_tiles();
    __syncthreads();
    if (kt + 1 < nk) load_tiles((kt + 1) * GBK);
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      bf16x8 af[MT], bfr[2];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        int m = wm * (BM / 2) + 32 * i + l32;
        af[i] = *reinterpret_cast<const bf16x8*>(&As[m * GBK + 8 * swz_a(m, 2 * ks + g)]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        int n = wn * 64 + 32 * j + l32;
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Bt[n * GBK + 8 * swz_b(n, 2 * ks + g)]);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)  // C^T tile: rows n, columns m
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  }

  if (EPI == 0) {
    // column sums of this block's 128 columns of W, summed over the 16 row
    // groups in a fixed order
#pragma unroll
    for (int j = 0; j < 8; ++j) colsum_part[(tid / 16) * GBN + 8 * (tid % 16) + j] = csum[j];
    __syncthreads();
    if (tid < GBN) {
      float s = 0.f;
      for (int q = 0; q < 16; ++q) s += colsum_part[q * GBN + tid];
      colsum_part[tid] = s;  // row 0 is read only after the barrier below
    }
    __syncthreads();
  }

  // epilogue: lane owns row m = ... + l32 and columns n = ... + 8 (r/4) + 4 g + [0, 4)
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = m0 + wm * (BM / 2) + 32 * i + l32;
    if (m >= M) continue;
    float mu = 0.f, rstd = 1.f;
    int64_t pool_row = -1;  // element offset of (page, head 0, slot) of row m, or -1
    if (EPI == 0) {
      float2 st = route.stats[m];
      mu = st.x;
      rstd = st.y;
      if (route.k_pool) {
        const int user = find_segment(route.new_offsets, route.B, m);
        const int pos = route.start_pos[user] + (m - route.new_offsets[user]);
        const int lp = pos / route.page_size;
        if (lp < route.max_pages) {
          const int page = route.page_table[static_cast<int64_t>(user) * route.max_pages + lp];
          if (page >= 0 && page < route.num_pages)
            pool_row = route.pool_layer_offset +
                       (static_cast<int64_t>(page) * route.H * route.page_size + (pos - lp * route.page_size)) *
                           route.dh;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // 32 columns starting at a multiple of 32: one chunk, one head (uniform)
      const int nb = n0 + wn * 64 + 32 * j;
      const int chunk = EPI == 0 ? nb / route.inner : 0;  // 0 U, 1 V, 2 Q, 3 K
      const int cb = nb - chunk * route.inner;
      const int h = EPI == 0 ? cb / route.dh : 0;
      const int e0 = cb - h * route.dh;
      const bool is_kv = EPI == 0 && (chunk == 1 || chunk == 3);
      const bool to_uvqk = EPI == 0 && (!is_kv || route.kv_to_uvqk || !route.k_pool);
      const bool to_pool = is_kv && pool_row >= 0;
      uint16_t* pool = chunk == 3 ? route.k_pool : route.v_pool;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * 64 + 32 * j + 8 * q + 4 * g;  // local column of the 4-group
        const int n = n0 + nl;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
        if (EPI == 0) {
          const f32x4 cs = *reinterpret_cast<const f32x4*>(&colsum_part[nl]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = rstd * (v[e] - mu * cs[e]);
            v[e] = z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.44269504088896340736f));
          }
        } else {
          const u32x2 r2 = *reinterpret_cast<const u32x2*>(R + static_cast<int64_t>(m) * N + n);
          v[0] += bf2f(r2[0] & 0xFFFFu);
          v[1] += bf2f(r2[0] >> 16);
          v[2] += bf2f(r2[1] & 0xFFFFu);
          v[3] += bf2f(r2[1] >> 16);
        }
        const u32x2 packed = {uint32_t(f2bf(v[0])) | (uint32_t(f2bf(v[1])) << 16),
                              uint32_t(f2bf(v[2])) | (uint32_t(f2bf(v[3])) << 16)};
        if (EPI == 1) {
          *reinterpret_cast<u32x2*>(C + static_cast<int64_t>(m) * N + n) = packed;
          continue;
        }
        if (to_uvqk) *reinterpret_cast<u32x2*>(route.uvqk + static_cast<int64_t>(m) * N + n) = packed;
        if (to_pool) {
          const int64_t off = pool_row + static_cast<int64_t>(h) * route.page_size * route.dh + e0 + 8 * q + 4 * g;
          *reinterpret_cast<u32x2*>(pool + off) = packed;
        }
      }
    }
  }
}

// per-row (mean, rstd) of x: one wave per row, two-pass from registers
constexpr int kStatRows = 4;
__global__ __launch_bounds__(64 * kStatRows) void row_stats_kernel(const uint16_t* __restrict__ x,
                                                                   float2* __restrict__ stats,
                                                                   int32_t rows, int32_t cols,
                                                                   float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kStatRows + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + static_cast<int64_t>(row) * cols;
  constexpr int kMaxChunks = 4;  // cols <= 64 * 8 * 4
  float v[kMaxChunks * 8];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int col = 8 * (lane + 64 * c);
    u32x4 raw = col < cols ? *reinterpret_cast<const u32x4*>(xr + col) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float f = bf2f(static_cast<uint16_t>((e & 1) ? (raw[e >> 1] >> 16) : (raw[e >> 1] & 0xFFFFu)));
      v[8 * c + e] = f;
      s += f;
    }
  }
  const float mean = wave_sum(s) / cols;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (8 * (lane + 64 * c) < cols) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float dv = v[8 * c + e] - mean;
        q += dv * dv;
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) / cols + eps);
  if (lane == 0) stats[row] = float2{mean, rstd};
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
      Bs[kb][nn] = (n < N && k2 < K) ? Bm[static_cast<int64_t>(k2) * N + n] : 0.f;
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

}  // namespace

hipError_t launch_row_stats(const void* x, float* stats, int32_t rows, int32_t cols, float eps,
                            hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (cols % 8 != 0 || cols > 64 * 8 * 4) return hipErrorInvalidValue;
  dim3 grid((rows + kStatRows - 1) / kStatRows), block(64 * kStatRows);
  hipLaunchKernelGGL(row_stats_kernel, grid, block, 0, s, static_cast<const uint16_t*>(x),
                     reinterpret_cast<float2*>(stats), rows, cols, eps);
  return hipGetLastError();
}

hipError_t launch_f1_bf16(const void* x, const float* stats, const void* w1, const F1Args& f,
                          int32_t M, int32_t N, int32_t K, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (N % GBN != 0 || K % GBK != 0 || f.inner % 32 != 0 || f.dh % 32 != 0) return hipErrorInvalidValue;
  F1Route r{};
  r.stats = reinterpret_cast<const float2*>(stats);
  r.uvqk = static_cast<uint16_t*>(f.uvqk);
  r.inner = f.inner;
  r.kv_to_uvqk = f.kv_to_uvqk;
  r.k_pool = static_cast<uint16_t*>(f.k_pool);
  r.v_pool = static_cast<uint16_t*>(f.v_pool);
  r.pool_layer_offset = f.pool_layer_offset;
  r.page_table = f.page_table;
  r.new_offsets = f.new_offsets;
  r.start_pos = f.start_pos;
  r.B = f.B;
  r.max_pages = f.max_pages;
  r.num_pages = f.num_pages;
  r.H = f.H;
  r.dh = f.dh;
  r.page_size = f.page_size;
  constexpr int BM = 128;
  dim3 grid(static_cast<unsigned>(((M + BM - 1) / BM) * (N / GBN)));
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, 0>), grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w1),
                     static_cast<uint16_t*>(f.uvqk), nullptr, r, M, N, K);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int epilogue, const void* A, const void* Bm, void* C,
                       const void* R, int32_t M, int32_t N, int32_t K, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (dtype == HSTU_BF16) {
    // the bf16 path only uses this for f2 (+ residual); f1 goes through launch_f1_bf16
    if (epilogue != 1 || N % GBN != 0 || K % GBK != 0) return hipErrorInvalidValue;
    constexpr int BM = 64;  // a short K loop: more blocks hide more load latency
    dim3 grid(static_cast<unsigned>(((M + BM - 1) / BM) * (N / GBN)));
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, 1>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bm),
                       static_cast<uint16_t*>(C), static_cast<const uint16_t*>(R), F1Route{}, M, N,
                       K);
  } else {
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

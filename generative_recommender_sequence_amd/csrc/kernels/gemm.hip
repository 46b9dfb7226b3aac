// The two projections of the HSTU layer ("How Generative Recommenders Are
// Redefining RecSys at Scale", section HSTU):
//   f1: [U|V|Q|K] = SiLU(x^ . W1)     (epilogue 0)
//   f2: y = x + g . W2                (epilogue 1)
// C[M][N] = epi(A[M][K] . B[K][N]), all row-major.
//
// bf16: 128x128 output tile per 256-thread block, 4 waves each owning 64x64
// as 2x2 v_mfma_f32_32x32x16_bf16 tiles, K staged 64 at a time through LDS.
// B is row-major [K][N] (the weight layout), but the MFMA B operand wants 8
// consecutive k per lane, so B tiles are written to LDS transposed (n-major).
// Both LDS tiles use a 16-byte-chunk XOR swizzle so that the transposing
// writes and the operand reads are free of bank conflicts.  The next K tile
// is fetched into registers while the current one is multiplied.
// Requires N % 128 == 0 and K % 64 == 0; M is arbitrary.
//
// fp32: a plain 64x64-tile FMA kernel (exact-ish reference precision path).
#include "common.h"

namespace hstu {
namespace {

constexpr int GBM = 128, GBN = 128, GBK = 64;

__device__ __forceinline__ float epi_silu(float x) { return x / (1.0f + __expf(-x)); }

__device__ __forceinline__ int swz_a(int m, int c) { return c ^ (m & 7); }
__device__ __forceinline__ int swz_b(int n, int c) { return c ^ ((n + (n >> 3)) & 7); }

template <int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ Bm,
                                                        uint16_t* __restrict__ C,
                                                        const uint16_t* __restrict__ R, int32_t M,
                                                        int32_t N, int32_t K) {
  __shared__ __attribute__((aligned(16))) uint16_t As[GBM * GBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bt[GBN * GBK];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_tiles_n = N / GBN;
  const int m0 = (blockIdx.x / n_tiles_n) * GBM;
  const int n0 = (blockIdx.x % n_tiles_n) * GBN;

  // global -> register staging: A 4 chunks (rows tid/8 + 32i, chunk tid%8);
  // B 2 rounds x 2 rows (k pair 2*(tid/16) + 32 r, n chunk tid%16)
  u32x4 ra[4], rb[4];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
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
    for (int i = 0; i < 4; ++i) {
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
        int n = nb + j;
        int chunk = swz_b(n, kk >> 3);
        *reinterpret_cast<uint32_t*>(&Bt[n * GBK + 8 * chunk + (kk & 7)]) = a | (b << 16);
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
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
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int m = wm * 64 + 32 * i + l32;
        af[i] = *reinterpret_cast<const bf16x8*>(&As[m * GBK + 8 * swz_a(m, 2 * ks + g)]);
        int n = wn * 64 + 32 * i + l32;
        bfr[i] = *reinterpret_cast<const bf16x8*>(&Bt[n * GBK + 8 * swz_b(n, 2 * ks + g)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: lane owns column l32 and rows 8(r/4) + 4g + r%4 of each 32x32 tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int n = n0 + wn * 64 + 32 * j + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        if (m < M) {
          int64_t idx = static_cast<int64_t>(m) * N + n;
          float v = acc[i][j][r];
          if (EPI == 0) v = epi_silu(v);
          else v += bf2f(R[idx]);
          C[idx] = f2bf(v);
        }
      }
    }
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

hipError_t launch_gemm(int dtype, int epilogue, const void* A, const void* Bm, void* C,
                       const void* R, int32_t M, int32_t N, int32_t K, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (dtype == HSTU_BF16) {
    if (N % GBN != 0 || K % GBK != 0) return hipErrorInvalidValue;
    dim3 grid(static_cast<unsigned>(((M + GBM - 1) / GBM) * (N / GBN)));
    auto a = static_cast<const uint16_t*>(A);
    auto b = static_cast<const uint16_t*>(Bm);
    auto c = static_cast<uint16_t*>(C);
    auto r = static_cast<const uint16_t*>(R);
    if (epilogue == 0)
      hipLaunchKernelGGL(gemm_bf16_kernel<0>, grid, dim3(256), 0, s, a, b, c, r, M, N, K);
    else
      hipLaunchKernelGGL(gemm_bf16_kernel<1>, grid, dim3(256), 0, s, a, b, c, r, M, N, K);
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

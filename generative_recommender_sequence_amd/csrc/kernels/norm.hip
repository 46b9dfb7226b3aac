// Row normalisations of the HSTU layer ("How Generative Recommenders Are
// Redefining RecSys at Scale", section HSTU: elementwise gating before the
// output projection):
//   pre-norm       x^ = LayerNorm(x) over d_model (no affine)
//   reduce + gate  o = (1/n_u) * sum of the row's partial attention tiles in
//                  key order; g = LayerNorm(o over all heads) * U
// One wave64 per row; statistics are two-pass from registers (mean, then the
// mean of squared deviations), reduced with cross-lane shuffles.
#include "common.h"

namespace hstu {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 waves
constexpr int kMaxPerLane = 32;   // row length <= 64 * 32

template <typename T>
__global__ __launch_bounds__(64 * kRowsPerBlock) void layer_norm_kernel(
    const T* __restrict__ x, T* __restrict__ y, int32_t rows, int32_t cols, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const T* xr = x + static_cast<int64_t>(row) * cols;
  float v[kMaxPerLane];
  float s = 0.f;
  int n = 0;
#pragma unroll
  for (int k = 0; k < kMaxPerLane; ++k) {
    int c = lane + 64 * k;
    v[k] = c < cols ? Elem<T>::load(xr + c) : 0.f;
    s += v[k];
  }
  (void)n;
  const float mean = wave_sum(s) / cols;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxPerLane; ++k) {
    int c = lane + 64 * k;
    float dv = c < cols ? v[k] - mean : 0.f;
    q += dv * dv;
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) / cols + eps);
  T* yr = y + static_cast<int64_t>(row) * cols;
#pragma unroll
  for (int k = 0; k < kMaxPerLane; ++k) {
    int c = lane + 64 * k;
    if (c < cols) Elem<T>::store(yr + c, (v[k] - mean) * rstd);
  }
}

// Each lane owns float4 chunks c = 4 * (lane + 64 k) of the row's H*dh values.
template <typename T>
__global__ __launch_bounds__(64 * kRowsPerBlock) void reduce_gate_kernel(
    PlanDev plan, const float* __restrict__ partials, float o_scale, const T* __restrict__ u,
    int64_t u_stride, float eps, float* __restrict__ o_out, T* __restrict__ g_out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= plan.n_new) return;
  const int dh = plan.dh, H = plan.H, inner = H * dh;
  const int qb = plan.row_qblock[row];
  const QBlock blk = plan.qblocks[qb];
  const int local = row - blk.row0;
  const float inv_n = plan.users[blk.user].inv_n * o_scale;
  constexpr int kChunks = kMaxPerLane / 4;  // inner <= 64 * 32
  f32x4 o[kChunks];
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    int c = 4 * (lane + 64 * k);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (c < inner) {
      int h = c / dh, e = c % dh;
      SlotRange sr = plan.qb_slots[qb * H + h];
      for (int s = 0; s < sr.count; ++s) {
        const float* p =
            partials + (static_cast<int64_t>(sr.first + s) * kBlockQ + local) * dh + e;
        acc += *reinterpret_cast<const f32x4*>(p);
      }
      acc *= inv_n;
    }
    o[k] = acc;
  }
  if (o_out) {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      int c = 4 * (lane + 64 * k);
      if (c < inner) *reinterpret_cast<f32x4*>(o_out + static_cast<int64_t>(row) * inner + c) = o[k];
    }
  }
  if (!g_out) return;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChunks; ++k) s += o[k][0] + o[k][1] + o[k][2] + o[k][3];
  const float mean = wave_sum(s) / inner;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    int c = 4 * (lane + 64 * k);
    if (c < inner) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float dv = o[k][j] - mean;
        q += dv * dv;
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) / inner + eps);
  const T* ur = u + static_cast<int64_t>(row) * u_stride;
  T* gr = g_out + static_cast<int64_t>(row) * inner;
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    int c = 4 * (lane + 64 * k);
    if (c < inner) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        Elem<T>::store(gr + c + j, (o[k][j] - mean) * rstd * Elem<T>::load(ur + c + j));
    }
  }
}

}  // namespace

hipError_t launch_layer_norm(int dtype, const void* x, void* xhat, int32_t rows, int32_t cols,
                             float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (cols > 64 * kMaxPerLane) return hipErrorInvalidValue;
  dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock), block(64 * kRowsPerBlock);
  if (dtype == HSTU_BF16)
    hipLaunchKernelGGL(layer_norm_kernel<uint16_t>, grid, block, 0, s,
                       static_cast<const uint16_t*>(x), static_cast<uint16_t*>(xhat), rows, cols, eps);
  else
    hipLaunchKernelGGL(layer_norm_kernel<float>, grid, block, 0, s, static_cast<const float*>(x),
                       static_cast<float*>(xhat), rows, cols, eps);
  return hipGetLastError();
}

hipError_t launch_reduce_gate(int dtype, const PlanDev& plan, const float* partials,
                              float o_scale, const void* u, int64_t u_stride, float eps,
                              float* o_out, void* g_out, hipStream_t s) {
  if (plan.n_new == 0) return hipSuccess;
  if (plan.H * plan.dh > 64 * kMaxPerLane) return hipErrorInvalidValue;
  dim3 grid((plan.n_new + kRowsPerBlock - 1) / kRowsPerBlock), block(64 * kRowsPerBlock);
  if (dtype == HSTU_BF16)
    hipLaunchKernelGGL(reduce_gate_kernel<uint16_t>, grid, block, 0, s, plan, partials, o_scale,
                       static_cast<const uint16_t*>(u), u_stride, eps, o_out,
                       static_cast<uint16_t*>(g_out));
  else
    hipLaunchKernelGGL(reduce_gate_kernel<float>, grid, block, 0, s, plan, partials, o_scale,
                       static_cast<const float*>(u), u_stride, eps, o_out,
                       static_cast<float*>(g_out));
  return hipGetLastError();
}

}  // namespace hstu

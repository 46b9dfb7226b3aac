// Row normalisations of the HSTU layer ("How Generative Recommenders Are
// Redefining RecSys at Scale", section HSTU: elementwise gating before the
// output projection):
//   pre-norm       x^ = LayerNorm(x) over d_model (no affine)
//   reduce + gate  o = (1/n_u) * sum of the row's partial attention tiles in
//                  key order (tiles stored in the layer's dtype, summed in
//                  fp32); g = LayerNorm(o over all heads) * U
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
// A block holds 4 rows of one q-block (blockIdx = q-block * 32 + row group),
// so the q-block and user records are block-uniform loads, the slot ranges
// depend only on the block and the lane's head, and the partial tiles are
// fetched four slots at a time (summed in slot order, i.e. key order).
constexpr int kGroups = kBlockQ / kRowsPerBlock;
// four consecutive values of a row as float (8- or 16-byte accesses)
__device__ __forceinline__ f32x4 load4(const uint16_t* p) {
  const u32x2 r = *reinterpret_cast<const u32x2*>(p);
  return f32x4{bf2f(r[0] & 0xFFFFu), bf2f(r[0] >> 16), bf2f(r[1] & 0xFFFFu), bf2f(r[1] >> 16)};
}
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void store4(uint16_t* p, f32x4 v) {
  *reinterpret_cast<u32x2*>(p) = u32x2{uint32_t(f2bf(v[0])) | (uint32_t(f2bf(v[1])) << 16),
                                       uint32_t(f2bf(v[2])) | (uint32_t(f2bf(v[3])) << 16)};
}
__device__ __forceinline__ void store4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
// four partial values as raw bits, widened once the round's loads are issued
__device__ __forceinline__ u32x2 load_raw4(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ f32x4 load_raw4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 widen4(u32x2 r) {
  return f32x4{bf2f(r[0] & 0xFFFFu), bf2f(r[0] >> 16), bf2f(r[1] & 0xFFFFu), bf2f(r[1] >> 16)};
}
__device__ __forceinline__ f32x4 widen4(f32x4 v) { return v; }
template <typename T, int kChunks>  // inner <= 64 * 4 * kChunks; U and g of type T, fp32 partials
__global__ __launch_bounds__(64 * kRowsPerBlock) void reduce_gate_kernel(
    PlanDev plan, const float* __restrict__ partials, float o_scale, const T* __restrict__ u,
    int64_t u_stride, float eps, float* __restrict__ o_out, T* __restrict__ g_out) {
  const int lane = threadIdx.x & 63;
  const int qb = blockIdx.x / kGroups;
  const int local = (blockIdx.x % kGroups) * kRowsPerBlock + (threadIdx.x >> 6);
  const int dh = plan.dh, H = plan.H, inner = H * dh;
  // slot ranges first: they need only the block and the lane's heads
  SlotRange sr[kChunks];
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int c = 4 * (lane + 64 * k);
    sr[k] = c < inner ? plan.qb_slots[qb * H + c / dh] : SlotRange{0, 0};
  }
  const QBlock blk = plan.qblocks[qb];
  if (local >= blk.count) return;
  const int row = blk.row0 + local;
  const float inv_n = plan.users[blk.user].inv_n * o_scale;
  // the gate's U, fetched while the partial tiles are summed (raw bits,
  // widened at use; lanes past the row re-read its last values)
  decltype(load_raw4(u)) uraw[kChunks];
  if (g_out) {
#pragma unroll
    for (int k = 0; k < kChunks; ++k)
      uraw[k] = load_raw4(u + static_cast<int64_t>(row) * u_stride + min(4 * (lane + 64 * k), inner - 4));
  }
  f32x4 o[kChunks];
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int c = 4 * (lane + 64 * k);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (c < inner) {
      const int e = c % dh;
      const float* p = partials + (static_cast<int64_t>(sr[k].first) * kBlockQ + local) * dh + e;
      const int64_t step = static_cast<int64_t>(kBlockQ) * dh;
      const int last = sr[k].count - 1;
      for (int s = 0; s <= last; s += 4) {
        // four loads issued together; past the last slot they re-read it and count zero
        const auto v0 = load_raw4(p + s * step);
        const auto v1 = load_raw4(p + min(s + 1, last) * step);
        const auto v2 = load_raw4(p + min(s + 2, last) * step);
        const auto v3 = load_raw4(p + min(s + 3, last) * step);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        acc += widen4(v0);
        acc += s + 1 <= last ? widen4(v1) : z;
        acc += s + 2 <= last ? widen4(v2) : z;
        acc += s + 3 <= last ? widen4(v3) : z;
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
  T* gr = g_out + static_cast<int64_t>(row) * inner;
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    int c = 4 * (lane + 64 * k);
    if (c < inner) store4(gr + c, (o[k] - mean) * rstd * widen4(uraw[k]));
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

hipError_t launch_reduce_gate(int dtype, const PlanDev& plan, const void* partials,
                              float o_scale, const void* u, int64_t u_stride, float eps,
                              float* o_out, void* g_out, hipStream_t s) {
  if (plan.n_new == 0) return hipSuccess;
  if (plan.H * plan.dh > 64 * kMaxPerLane) return hipErrorInvalidValue;
  if (plan.n_qblocks == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(plan.n_qblocks) * kGroups), block(64 * kRowsPerBlock);
  const bool narrow = plan.H * plan.dh <= 64 * 4 * 2;  // the configurations' 512 values a row
  auto* pp = static_cast<const float*>(partials);
  if (dtype == HSTU_BF16) {
    auto* uu = static_cast<const uint16_t*>(u);
    auto* gg = static_cast<uint16_t*>(g_out);
    if (narrow)
      hipLaunchKernelGGL((reduce_gate_kernel<uint16_t, 2>), grid, block, 0, s, plan, pp, o_scale, uu, u_stride,
                         eps, o_out, gg);
    else
      hipLaunchKernelGGL((reduce_gate_kernel<uint16_t, kMaxPerLane / 4>), grid, block, 0, s, plan, pp, o_scale,
                         uu, u_stride, eps, o_out, gg);
  } else {
    auto* uu = static_cast<const float*>(u);
    auto* gg = static_cast<float*>(g_out);
    if (narrow)
      hipLaunchKernelGGL((reduce_gate_kernel<float, 2>), grid, block, 0, s, plan, pp, o_scale, uu, u_stride,
                         eps, o_out, gg);
    else
      hipLaunchKernelGGL((reduce_gate_kernel<float, kMaxPerLane / 4>), grid, block, 0, s, plan, pp, o_scale, uu,
                         u_stride, eps, o_out, gg);
  }
  return hipGetLastError();
}

}  // namespace hstu

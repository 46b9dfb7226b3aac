// Byte-exact movement of K/V rows between token-major buffers and the paged
// KV table ("Deploying an HSTU Generative Recommender with NVIDIA
// Dynamo-Triton", KV cache section: the paged table supports append; the
// attention consumes the cached data directly).
//
// Pool layout: [layer][page][head][slot][head_dim], so one head's page is a
// contiguous page_size * head_dim block.  Each thread moves one 16-byte chunk
// of K and the matching chunk of V.  Page ids outside [0, num_pages) and
// positions past the page table are skipped rather than dereferenced.
#include "common.h"

namespace hstu {
namespace {

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void append_kernel(
    int32_t B, const int32_t* __restrict__ new_off, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ page_table, int32_t max_pages, const char* __restrict__ k_new,
    const char* __restrict__ v_new, int64_t row_stride_bytes, int64_t n_chunks,
    int32_t chunks_per_row, int32_t chunks_per_head, char* __restrict__ k_pool,
    char* __restrict__ v_pool, int64_t layer_off_bytes, int32_t num_pages, int32_t H,
    int32_t page_size, int32_t head_bytes) {
  int64_t id = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
  if (id >= n_chunks) return;
  int32_t r = static_cast<int32_t>(id / chunks_per_row);
  int32_t c = static_cast<int32_t>(id % chunks_per_row);
  int32_t h = c / chunks_per_head, ch = c % chunks_per_head;
  int u = find_segment(new_off, B, r);
  int32_t pos = start_pos[u] + (r - new_off[u]);
  int32_t lp = pos / page_size;
  if (pos < 0 || lp >= max_pages) return;
  int32_t page = page_table[static_cast<int64_t>(u) * max_pages + lp];
  if (page < 0 || page >= num_pages) return;
  int64_t dst = layer_off_bytes +
                ((static_cast<int64_t>(page) * H + h) * page_size + pos % page_size) * head_bytes +
                ch * 16;
  int64_t src = r * row_stride_bytes + static_cast<int64_t>(h) * head_bytes + ch * 16;
  u32x4 kv = *reinterpret_cast<const u32x4*>(k_new + src);
  u32x4 vv = *reinterpret_cast<const u32x4*>(v_new + src);
  *reinterpret_cast<u32x4*>(k_pool + dst) = kv;
  *reinterpret_cast<u32x4*>(v_pool + dst) = vv;
}

__global__ __launch_bounds__(kCopyThreads) void gather_kernel(
    int32_t B, const int32_t* __restrict__ page_table, int32_t max_pages,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ out_off, int64_t n_chunks,
    int32_t chunks_per_row, int32_t chunks_per_head, char* __restrict__ k_out,
    char* __restrict__ v_out, const char* __restrict__ k_pool, const char* __restrict__ v_pool,
    int64_t layer_off_bytes, int32_t num_pages, int32_t H, int32_t page_size, int32_t head_bytes) {
  int64_t id = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
  if (id >= n_chunks) return;
  int32_t r = static_cast<int32_t>(id / chunks_per_row);
  int32_t c = static_cast<int32_t>(id % chunks_per_row);
  int32_t h = c / chunks_per_head, ch = c % chunks_per_head;
  int u = find_segment(out_off, B, r);
  int32_t pos = r - out_off[u];
  if (pos >= kv_len[u]) return;
  int32_t lp = pos / page_size;
  if (lp >= max_pages) return;
  int32_t page = page_table[static_cast<int64_t>(u) * max_pages + lp];
  if (page < 0 || page >= num_pages) return;
  int64_t src = layer_off_bytes +
                ((static_cast<int64_t>(page) * H + h) * page_size + pos % page_size) * head_bytes +
                ch * 16;
  int64_t dst = static_cast<int64_t>(r) * chunks_per_row * 16 + static_cast<int64_t>(c) * 16;
  *reinterpret_cast<u32x4*>(k_out + dst) = *reinterpret_cast<const u32x4*>(k_pool + src);
  *reinterpret_cast<u32x4*>(v_out + dst) = *reinterpret_cast<const u32x4*>(v_pool + src);
}

}  // namespace

hipError_t launch_append(int dtype, const PlanDev*, int32_t B, const int32_t* d_new_offsets,
                         const int32_t* d_start_pos, const int32_t* d_page_table, int32_t max_pages,
                         const void* k_new, const void* v_new, int64_t row_stride,
                         int32_t n_new_total, void* k_pool, void* v_pool, int32_t layer,
                         int32_t num_pages, int32_t H, int32_t dh, int32_t page_size,
                         hipStream_t s) {
  const int es = dtype == HSTU_BF16 ? 2 : 4;
  const int head_bytes = dh * es;
  const int cph = head_bytes / 16, cpr = cph * H;
  const int64_t n_chunks = static_cast<int64_t>(n_new_total) * cpr;
  if (n_chunks == 0) return hipSuccess;
  const int64_t layer_off = static_cast<int64_t>(layer) * num_pages * H * page_size * head_bytes;
  dim3 grid(static_cast<unsigned>((n_chunks + kCopyThreads - 1) / kCopyThreads));
  hipLaunchKernelGGL(append_kernel, grid, dim3(kCopyThreads), 0, s, B, d_new_offsets, d_start_pos,
                     d_page_table, max_pages, static_cast<const char*>(k_new),
                     static_cast<const char*>(v_new), row_stride * es, n_chunks, cpr, cph,
                     static_cast<char*>(k_pool), static_cast<char*>(v_pool), layer_off, num_pages,
                     H, page_size, head_bytes);
  return hipGetLastError();
}

hipError_t launch_gather(int dtype, int32_t B, const int32_t* d_page_table, int32_t max_pages,
                         const int32_t* d_kv_len, const int32_t* d_out_offsets, int32_t n_out_total,
                         void* k_out, void* v_out, const void* k_pool, const void* v_pool,
                         int32_t layer, int32_t num_pages, int32_t H, int32_t dh, int32_t page_size,
                         hipStream_t s) {
  const int es = dtype == HSTU_BF16 ? 2 : 4;
  const int head_bytes = dh * es;
  const int cph = head_bytes / 16, cpr = cph * H;
  const int64_t n_chunks = static_cast<int64_t>(n_out_total) * cpr;
  if (n_chunks == 0) return hipSuccess;
  const int64_t layer_off = static_cast<int64_t>(layer) * num_pages * H * page_size * head_bytes;
  dim3 grid(static_cast<unsigned>((n_chunks + kCopyThreads - 1) / kCopyThreads));
  hipLaunchKernelGGL(gather_kernel, grid, dim3(kCopyThreads), 0, s, B, d_page_table, max_pages,
                     d_kv_len, d_out_offsets, n_chunks, cpr, cph, static_cast<char*>(k_out),
                     static_cast<char*>(v_out), static_cast<const char*>(k_pool),
                     static_cast<const char*>(v_pool), layer_off, num_pages, H, page_size,
                     head_bytes);
  return hipGetLastError();
}

namespace {
// One block per (page pair, layer, K or V): a whole page of all heads, 16
// bytes per lane per step.
__global__ __launch_bounds__(256) void tier_copy_kernel(const PagePair* __restrict__ pairs, int32_t layers,
                                                       const u32x4* __restrict__ sk, const u32x4* __restrict__ sv,
                                                       int64_t src_pages, u32x4* __restrict__ dk,
                                                       u32x4* __restrict__ dv, int64_t dst_pages,
                                                       int64_t page_chunks) {
  int64_t idx = blockIdx.x;
  const int kv = static_cast<int>(idx & 1);
  idx >>= 1;
  const int64_t layer = idx % layers;
  const PagePair pp = pairs[idx / layers];
  const u32x4* src = (kv ? sv : sk) + (layer * src_pages + pp.src) * page_chunks;
  u32x4* dst = (kv ? dv : dk) + (layer * dst_pages + pp.dst) * page_chunks;
  for (int64_t i = threadIdx.x; i < page_chunks; i += blockDim.x) dst[i] = src[i];
}
}  // namespace

hipError_t launch_tier_copy(const PagePair* pairs, int32_t n_pairs, int32_t layers, const void* src_k,
                            const void* src_v, int64_t src_pages, void* dst_k, void* dst_v,
                            int64_t dst_pages, int64_t page_bytes, hipStream_t s) {
  if (n_pairs == 0 || layers == 0) return hipSuccess;
  if (page_bytes % 16 != 0) return hipErrorInvalidValue;
  const int64_t blocks = static_cast<int64_t>(n_pairs) * layers * 2;
  hipLaunchKernelGGL(tier_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, pairs, layers,
                     static_cast<const u32x4*>(src_k), static_cast<const u32x4*>(src_v), src_pages,
                     static_cast<u32x4*>(dst_k), static_cast<u32x4*>(dst_v), dst_pages, page_bytes / 16);
  return hipGetLastError();
}

}  // namespace hstu

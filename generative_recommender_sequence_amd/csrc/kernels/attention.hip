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
// fp32 partial tile, and the reduction adds the tiles of a row in key order,
// so the result does not depend on scheduling.
//
// bf16 kernel (gfx950, 256 threads = 4 waves, 32 queries per wave):
//   S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 (keys are the M rows, queries
//   the N columns), so after SiLU each lane already holds, for its own query,
//   the 8 key weights that form one A operand of O += P . V.  V is staged in
//   LDS transposed ([dh][key]) with the key order permuted inside each
//   16-key group (bits 2 and 3 swapped) so a B operand is one 16-byte read;
//   rows are XOR-swizzled by 16-byte chunk to keep both the transposing
//   writes and the reads free of bank conflicts.  The bias of a tile comes
//   from a reversed per-tile table in LDS read with immediate offsets, or from
//   one scalar when a wave's whole distance range falls in a single bucket.
//   Masking work is only done on tiles that touch the diagonal or the
//   candidate block.
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

__device__ __forceinline__ float rab_at(const float* rab, int nb, int delta) {
  return delta < 0 ? 0.f : rab[rel_bucket(delta, nb)];
}

// position inside a 16-key group of LDS V^T: swap key bits 2 and 3
__device__ __forceinline__ int vperm(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}
__device__ __forceinline__ int vswz(int d, int chunk) { return chunk ^ ((d + (d >> 3)) & 7); }

template <bool PAGED>
__device__ __forceinline__ const uint16_t* kv_row(const AttnLaunch& a, const uint16_t* base,
                                                  const UserInfo& ui, int user, int h, int j) {
  if (PAGED) {
    const int P = a.plan.page_size;
    int lp = j / P;
    if (lp >= a.plan.max_pages) return nullptr;
    int page = a.page_table[static_cast<int64_t>(user) * a.plan.max_pages + lp];
    if (page < 0 || page >= a.num_pages) return nullptr;
    return base + a.pool_layer_offset +
           ((static_cast<int64_t>(page) * a.plan.H + h) * P + (j % P)) * DH;
  } else {
    return base + static_cast<int64_t>(ui.kv_row0 + j) * a.kv_stride + h * DH;
  }
}

template <bool PAGED>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnLaunch a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DH * KT];
  __shared__ float bias_rev[256];

  const WorkItem w = a.plan.items[blockIdx.x];
  const QBlock qb = a.plan.qblocks[w.qblock];
  const UserInfo ui = a.plan.users[w.user];
  const int h = w.head;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wq0 = wave * 32;                 // first local query of this wave
  const bool wave_active = wq0 < qb.count;
  const int qlocal = wq0 + l32;
  const int qpos = qb.pos0 + qlocal;         // sequence position of this lane's query
  const int qa = qb.pos0, qe = qb.pos0 + qb.count;
  const int hist = ui.hist;
  const int nb = a.num_buckets;

  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);
  const uint16_t* kbase = static_cast<const uint16_t*>(PAGED ? a.k_pool : a.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(PAGED ? a.v_pool : a.v);

  // Q^T as the B operand of S^T = K . Q^T: lane holds q[query l32][16 s + 8 g .. +8]
  bf16x8 qf[DH / 16];
  {
    const bool qv = qlocal < qb.count;
    const uint16_t* qrow = qbase + static_cast<int64_t>(qb.row0 + (qv ? qlocal : 0)) * a.q_stride + h * DH;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      u32x4 raw = qv ? *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * g) : u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 oacc[DH / 32];
#pragma unroll
  for (int t = 0; t < DH / 32; ++t) oacc[t] = f32x16{};

  // loader roles: K rows key = tid/16 + 16 i, 16-byte chunk tid%16;
  // V: chunk dc = tid%16 (dims 8dc..8dc+7), keys 4*(tid/16) .. +3
  const int lc = tid & 15, lr = tid >> 4;

  for (int tile = w.tile_begin; tile < w.tile_end; ++tile) {
    const int k0 = tile * KT;
    if (!tile_visible_dev(k0, qa, qe, hist)) continue;  // uniform over the block
    __syncthreads();  // previous tile's LDS reads are done
    // ---- stage K (row-major) and V^T (permuted, swizzled) ----
#pragma unroll
    for (int i = 0; i < KT / 16; ++i) {
      int key = lr + 16 * i;
      int j = k0 + key;
      const uint16_t* src = j < ui.kv_len ? kv_row<PAGED>(a, kbase, ui, w.user, h, j) : nullptr;
      u32x4 v = src ? *reinterpret_cast<const u32x4*>(src + 8 * lc) : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&Ks[key * DH + 8 * (lc ^ (key & 7))]) = v;
    }
    {
      u32x4 vr[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        int j = k0 + 4 * lr + m;
        const uint16_t* src = j < ui.kv_len ? kv_row<PAGED>(a, vbase, ui, w.user, h, j) : nullptr;
        vr[m] = src ? *reinterpret_cast<const u32x4*>(src + 8 * lc) : u32x4{0u, 0u, 0u, 0u};
      }
      const int pos = vperm(4 * lr);  // 4 consecutive keys stay consecutive
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int d = 8 * lc + e;
        uint32_t w0 = (e & 1) ? (vr[0][e >> 1] >> 16) : (vr[0][e >> 1] & 0xFFFFu);
        uint32_t w1 = (e & 1) ? (vr[1][e >> 1] >> 16) : (vr[1][e >> 1] & 0xFFFFu);
        uint32_t w2 = (e & 1) ? (vr[2][e >> 1] >> 16) : (vr[2][e >> 1] & 0xFFFFu);
        uint32_t w3 = (e & 1) ? (vr[3][e >> 1] >> 16) : (vr[3][e >> 1] & 0xFFFFu);
        u32x2 pk = {w0 | (w1 << 16), w2 | (w3 << 16)};
        int chunk = vswz(d, pos >> 3);
        *reinterpret_cast<u32x2*>(&Vt[d * KT + 8 * chunk + (pos & 7)]) = pk;
      }
    }
    // ---- reversed bias table: bias_rev[t] = rab(b(delta_hi - t)) ----
    const int delta_hi = qa + BQ - 1 - k0;
    if (tid < kBiasLen) bias_rev[tid] = rab_at(a.rab, nb, delta_hi - tid);
    __syncthreads();
    if (!wave_active) continue;

    // ---- S^T = K . Q^T ----
    f32x16 sacc[KT / 32];
#pragma unroll
    for (int mt = 0; mt < KT / 32; ++mt) {
      sacc[mt] = f32x16{};
      int key = 32 * mt + l32;
#pragma unroll
      for (int s = 0; s < DH / 16; ++s) {
        bf16x8 kf = *reinterpret_cast<const bf16x8*>(&Ks[key * DH + 8 * ((2 * s + g) ^ (key & 7))]);
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[mt], 0, 0, 0);
      }
    }

    // ---- bias, mask, SiLU ----
    // lane's keys: k0 + 32 mt + 8 (r/4) + 4 g + (r%4); distance qpos - key
    const int wq_lo = qa + wq0, wq_hi = qa + wq0 + 31;
    const int dmin = wq_lo - (k0 + KT - 1), dmax = wq_hi - k0;
    const bool full = (k0 + KT - 1 < wq_lo) && (k0 + KT - 1 < hist);  // no masking needed
    const bool uni = dmin >= 0 && rel_bucket(dmin, nb) == rel_bucket(dmax, nb);
    const float ubias = uni ? a.rab[rel_bucket(dmax, nb)] : 0.f;
    const float* brow = &bias_rev[BQ - 1 - qlocal + 4 * g];  // + 32 mt + 8 (r/4) + r%4
#pragma unroll
    for (int mt = 0; mt < KT / 32; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int koff = 32 * mt + 8 * (r >> 2) + (r & 3);
        float x = sacc[mt][r] + (uni ? ubias : brow[koff]);
        float p = silu_fast(x);
        if (!full) {
          const int key = k0 + koff + 4 * g;
          const bool vis = (key == qpos) || (key < qpos && key < hist);
          p = vis ? p : 0.f;
        }
        sacc[mt][r] = p;
      }
    }

    // ---- O += P . V ----
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      const f32x16& src = sacc[ks >> 1];
      const int base = 8 * (ks & 1);
      bf16x8 pa;
#pragma unroll
      for (int e = 0; e < 8; ++e) pa[e] = static_cast<__bf16>(src[base + e]);
#pragma unroll
      for (int nt = 0; nt < DH / 32; ++nt) {
        int d = 32 * nt + l32;
        bf16x8 vb = *reinterpret_cast<const bf16x8*>(&Vt[d * KT + 8 * vswz(d, 2 * ks + g)]);
        oacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vb, oacc[nt], 0, 0, 0);
      }
    }
  }

  if (!wave_active) return;
  // ---- partial tile [BQ][DH] fp32: lane holds column 32 nt + l32, rows 8(r/4)+4g+r%4 ----
  float* out = a.partials + static_cast<int64_t>(w.slot) * BQ * DH;
#pragma unroll
  for (int nt = 0; nt < DH / 32; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int row = wq0 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (row < qb.count) out[row * DH + 32 * nt + l32] = oacc[nt][r];
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
  const QBlock qb = a.plan.qblocks[w.qblock];
  const UserInfo ui = a.plan.users[w.user];
  const int h = w.head, tid = threadIdx.x;
  const int qpos = qb.pos0 + tid;
  const bool qv = tid < qb.count;
  const float* qbase = static_cast<const float*>(a.q);
  const float* kbase = static_cast<const float*>(PAGED ? a.k_pool : a.k);
  const float* vbase = static_cast<const float*>(PAGED ? a.v_pool : a.v);
  float q[D], o[D];
  for (int e = 0; e < D; ++e) {
    q[e] = qv ? qbase[static_cast<int64_t>(qb.row0 + tid) * a.q_stride + h * D + e] : 0.f;
    o[e] = 0.f;
  }
  const int qa = qb.pos0, qe = qb.pos0 + qb.count;
  for (int tile = w.tile_begin; tile < w.tile_end; ++tile) {
    if (!tile_visible_dev(tile * KT, qa, qe, ui.hist)) continue;
    for (int sub = 0; sub < KT; sub += SK) {
      const int k0 = tile * KT + sub;
      __syncthreads();
      for (int i = tid; i < SK * D; i += 128) {
        int kk = i / D, e = i % D, j = k0 + kk;
        const float* kr = nullptr;
        const float* vr = nullptr;
        if (j < ui.kv_len) {
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
            kr = kbase + static_cast<int64_t>(ui.kv_row0 + j) * a.kv_stride + h * D;
            vr = vbase + static_cast<int64_t>(ui.kv_row0 + j) * a.kv_stride + h * D;
          }
        }
        Ks[kk][e] = kr ? kr[e] : 0.f;
        Vs[kk][e] = vr ? vr[e] : 0.f;
      }
      __syncthreads();
      if (!qv) continue;
      for (int kk = 0; kk < SK; ++kk) {
        const int j = k0 + kk;
        const bool vis = (j == qpos) || (j < qpos && j < ui.hist);
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
  float* out = a.partials + (static_cast<int64_t>(w.slot) * BQ + tid) * D;
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

// Stand-ins for the library's kernel launchers, for a host-only build of
// its C++ (cache manager, batcher, request planner, ABI validation) under
// AddressSanitizer and UndefinedBehaviorSanitizer.  That build runs the
// host-logic tests only; every launcher here reports that no kernel was
// launched, so a device call through it fails with HSTU_ERR_DEVICE.
#include "../../generative_recommender_sequence_amd/csrc/internal.h"

namespace hstu {
namespace {
hipError_t none() { return hipErrorNotSupported; }
}  // namespace

hipError_t launch_append(int, const PlanDev*, int32_t, const int32_t*, const int32_t*, const int32_t*, int32_t,
                         const void*, const void*, int64_t, int32_t, void*, void*, int32_t, int32_t, int32_t, int32_t,
                         int32_t, hipStream_t) { return none(); }
hipError_t launch_tier_copy(const PagePair*, int32_t, int32_t, const void*, const void*, int64_t, void*, void*, int64_t,
                            int64_t, hipStream_t) { return none(); }
hipError_t launch_gather(int, int32_t, const int32_t*, int32_t, const int32_t*, const int32_t*, int32_t, void*, void*,
                         const void*, const void*, int32_t, int32_t, int32_t, int32_t, int32_t, hipStream_t) {
  return none();
}
hipError_t launch_attention(const AttnLaunch&, hipStream_t) { return none(); }
hipError_t launch_reduce_gate(int, const PlanDev&, const void*, float, const void*, int64_t, float, float*, void*,
                              hipStream_t) { return none(); }
hipError_t launch_layer_norm(int, const void*, void*, int32_t, int32_t, float, hipStream_t) { return none(); }
hipError_t launch_gemm(int, int, const void*, const void*, void*, const void*, int32_t, int32_t, int32_t, hipStream_t,
                       RowStat*) { return none(); }
hipError_t launch_row_stats(const void*, RowStat*, int32_t, int32_t, const void*, float*, int32_t, const RowSlots&,
                            hipStream_t) { return none(); }
hipError_t launch_f1_bf16(const void*, const RowStat*, int32_t, const float*, const void*, const F1Args&, int32_t,
                          int32_t, int32_t, hipStream_t) { return none(); }
hipError_t launch_head_bf16(const HeadArgs&, hipStream_t) { return none(); }
hipError_t launch_attn_bwd(const BwdLaunch&, hipStream_t) { return none(); }
hipError_t launch_drab_sum(const float*, int32_t, int32_t, float*, hipStream_t) { return none(); }
hipError_t launch_gate_bwd(const float*, const void*, int64_t, const void*, int32_t, int32_t, float, void*, void*,
                           void*, hipStream_t) { return none(); }
hipError_t launch_ln_bwd(const void*, const void*, const void*, int32_t, int32_t, float, void*, void*, hipStream_t) {
  return none();
}
hipError_t launch_silu_grad(void*, const void*, int64_t, hipStream_t) { return none(); }
hipError_t launch_fill_zero(void*, int32_t, hipStream_t) { return none(); }
hipError_t launch_wgrad(const void*, int64_t, const void*, int64_t, int32_t, int32_t, int32_t, int32_t, const void*,
                        float*, float*, hipStream_t) { return none(); }
hipError_t launch_ceiling_mfma(int32_t, int32_t, float*, hipStream_t) { return none(); }
hipError_t launch_ceiling_read(const void*, int64_t, void*, hipStream_t) { return none(); }
hipError_t launch_ceiling_copy(const void*, void*, int64_t, hipStream_t) { return none(); }
}  // namespace hstu

extern "C" {
hstu_status hstu_attn_fwd_static(const hstu_attn_args*, hipStream_t) {
  return hstu::fail(HSTU_ERR_UNSUPPORTED, "hstu_attn_fwd_static: not in the host-only build");
}
size_t hstu_attn_static_scratch_bytes(void) { return 0; }
}

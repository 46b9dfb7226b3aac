// Event timing of the library's kernel launches (hstu_timing_enable /
// hstu_timing_read): a start and an end event on the launch stream around
// each kernel, so durations are measured on the stream the kernel runs on.
#include <cstring>
#include <mutex>
#include <utility>

#include "internal.h"

namespace hstu {
namespace {

const char* kNames[TK_COUNT] = {"layer_norm", "f1_gemm",  "append", "attention",
                                "reduce_gate", "f2_gemm", "gather", "head",
                                "bwd_attention", "bwd_gemm", "bwd_rows", "attention_cached",
                                "attention_prefill"};

struct TimingState {
  std::mutex mu;
  bool enabled = false;
  int mode = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> recs[TK_COUNT];
  std::vector<hipEvent_t> spare;

  hipEvent_t get() {
    if (!spare.empty()) {
      hipEvent_t e = spare.back();
      spare.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void clear() {
    for (auto& v : recs) {
      for (auto& p : v) {
        spare.push_back(p.first);
        spare.push_back(p.second);
      }
      v.clear();
    }
  }
};

TimingState& state() {
  static TimingState s;
  return s;
}

}  // namespace

int timing_mode() {
  TimingState& st = state();
  std::lock_guard<std::mutex> lk(st.mu);
  return st.mode;
}

TimedLaunch::TimedLaunch(TimedKernel k, hipStream_t s) : kernel(k), stream(s), start_ev(nullptr) {
  TimingState& st = state();
  std::lock_guard<std::mutex> lk(st.mu);
  if (!st.enabled) return;
  hipEvent_t e = st.get();
  if (e && hipEventRecord(e, s) == hipSuccess) start_ev = e;
}

void TimedLaunch::end() {
  if (!start_ev) return;
  TimingState& st = state();
  std::lock_guard<std::mutex> lk(st.mu);
  hipEvent_t e = st.get();
  if (e && hipEventRecord(e, stream) == hipSuccess)
    st.recs[kernel].emplace_back(static_cast<hipEvent_t>(start_ev), e);
  start_ev = nullptr;
}

}  // namespace hstu

using namespace hstu;

extern "C" {

hstu_status hstu_timing_enable(int32_t enable) {
  TimingState& st = state();
  std::lock_guard<std::mutex> lk(st.mu);
  st.clear();
  st.enabled = enable != 0;
  st.mode = enable == 2 ? 2 : (enable != 0 ? 1 : 0);
  // events made up front, so that recording them costs no creation on the launch path
  while (st.enabled && st.spare.size() < 4096) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) break;
    st.spare.push_back(e);
  }
  return ok();
}

hstu_status hstu_ceiling_mfma(int32_t blocks, int32_t iters, float* out, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || !out) return fail(HSTU_ERR_INVALID, "hstu_ceiling_mfma: bad argument");
  return check_hip(launch_ceiling_mfma(blocks, iters, out, stream), "hstu_ceiling_mfma");
}

hstu_status hstu_ceiling_read(const void* src, int64_t bytes, void* out, hipStream_t stream) {
  if (!src || !out || bytes <= 0 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return fail(HSTU_ERR_INVALID, "hstu_ceiling_read: bad argument");
  return check_hip(launch_ceiling_read(src, bytes, out, stream), "hstu_ceiling_read");
}

hstu_status hstu_ceiling_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 ||
      reinterpret_cast<uintptr_t>(dst) % 16)
    return fail(HSTU_ERR_INVALID, "hstu_ceiling_copy: bad argument");
  return check_hip(launch_ceiling_copy(src, dst, bytes, stream), "hstu_ceiling_copy");
}

hstu_status hstu_timing_read(const char* kernel, int32_t* launches, double* total_ms) {
  if (!kernel || !launches || !total_ms) return fail(HSTU_ERR_INVALID, "hstu_timing_read: null argument");
  int k = -1;
  for (int i = 0; i < TK_COUNT; ++i)
    if (std::strcmp(kernel, kNames[i]) == 0) k = i;
  if (k < 0) return fail(HSTU_ERR_INVALID, "hstu_timing_read: unknown kernel name");
  TimingState& st = state();
  std::lock_guard<std::mutex> lk(st.mu);
  double sum = 0.0;
  for (auto& p : st.recs[k]) {
    hstu_status s2 = check_hip(hipEventSynchronize(p.second), "hstu_timing_read");
    if (s2 != HSTU_OK) return s2;
    float ms = 0.f;
    if ((s2 = check_hip(hipEventElapsedTime(&ms, p.first, p.second), "hstu_timing_read")) != HSTU_OK)
      return s2;
    sum += ms;
  }
  *launches = static_cast<int32_t>(st.recs[k].size());
  *total_ms = sum;
  for (auto& p : st.recs[k]) {
    st.spare.push_back(p.first);
    st.spare.push_back(p.second);
  }
  st.recs[k].clear();
  return ok();
}

}  // extern "C"

// hstu_attn_fwd_static: the attention call for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid allocation).  It runs the same kernels as hstu_attn_fwd, but
// the fp32 partial tiles of the split-key attention live in a library-owned
// static device array instead of a caller workspace.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In
// host code its name is only a stand-in, so its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and kept;
// kernels receive that address.  Calls on one device share the array and it
// keeps the last call's contents: each call writes every partial it reads
// before reading it, so nothing needs clearing, but calls that overlap on one
// device (two streams, or two host threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace hstu {
namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(128) << 20;  // 2048 partial tiles at head_dim 128
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchAddresses {
  std::mutex mu;
  void* dev[kMaxDevices] = {};
};

ScratchAddresses& addresses() {
  static ScratchAddresses a;
  return a;
}

// Device address of this device's copy of the array, looked up on first use.
hstu_status scratch_address(void** out) {
  int dev = -1;
  hstu_status st = check_hip(hipGetDevice(&dev), "hstu_attn_fwd_static: current device");
  if (st != HSTU_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(HSTU_ERR_UNSUPPORTED, "hstu_attn_fwd_static: device index above 63");
  ScratchAddresses& a = addresses();
  std::lock_guard<std::mutex> lk(a.mu);
  if (!a.dev[dev]) {
    void* p = nullptr;
    st = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hstu_attn_fwd_static: scratch address");
    if (st != HSTU_OK) return st;
    if (!p) return fail(HSTU_ERR_DEVICE, "hstu_attn_fwd_static: scratch address is null");
    a.dev[dev] = p;
  }
  *out = a.dev[dev];
  return HSTU_OK;
}

}  // namespace
}  // namespace hstu

using namespace hstu;

extern "C" {

size_t hstu_attn_static_scratch_bytes(void) { return kScratchBytes; }

hstu_status hstu_attn_fwd_static(const hstu_attn_args* a, hipStream_t stream) {
  if (!a || !a->plan) return fail(HSTU_ERR_INVALID, "hstu_attn_fwd_static: null args or plan");
  hstu_plan_info info{};
  hstu_status st = hstu_plan_get_info(a->plan, &info);
  if (st != HSTU_OK) return st;
  if (info.attn_workspace_bytes > kScratchBytes)
    return fail(HSTU_ERR_UNSUPPORTED, "hstu_attn_fwd_static: the plan's partial tiles (" +
                                          std::to_string(info.attn_workspace_bytes) + " bytes) exceed the " +
                                          std::to_string(kScratchBytes) + "-byte static scratch");
  void* p = nullptr;
  if ((st = scratch_address(&p)) != HSTU_OK) return st;
  return attn_fwd_into(a, p, kScratchBytes, stream, "hstu_attn_fwd_static");
}

}  // extern "C"

// pa_forward without allocation: the partial-result workspace lives in a
// static device array instead of caller memory, for callers that cannot call
// hipMalloc (code under graph capture, tight serving loops, harnesses that
// forbid allocation).  The kernels are pa_forward's; only the workspace
// pointer differs.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "internal.h"

namespace {

// Largest workspace the static array holds.  Partial records take
// (head_size + 1) * 4 bytes per (record, query head); 64 MiB covers, e.g.,
// 3,900 records of 32 heads at head size 128.  Every device the library runs
// on holds one copy until the process ends.
constexpr size_t kScratchBytes = size_t(64) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` per device, looked up on the first call made
// for a plan of that device (the array's host-side name is not a device
// address).
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

pa_status scratch_of(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return pa::set_last_error(PA_ERR_INVALID_ARG, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev && hipSetDevice(dev) != hipSuccess)
      return pa::set_last_error(PA_ERR_HIP, "hipSetDevice failed");
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (prev >= 0 && prev != dev) (void)hipSetDevice(prev);
    if (e != hipSuccess || !ptr)
      return pa::set_last_error(PA_ERR_HIP, std::string("hipGetSymbolAddress: ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_forward_noalloc(const pa_plan* plan, const void* q, const void* kv_cache,
                                        const int32_t* block_table, const int32_t* query_start_loc,
                                        const int32_t* seq_lens, void* out, float* lse, void* stream) {
  pa::set_last_error(PA_OK, "");
  if (!plan) return pa::set_last_error(PA_ERR_INVALID_ARG, "plan is NULL");
  const int dev = pa::plan_device(plan);
  if (dev < 0) return pa::set_last_error(PA_ERR_INVALID_ARG, "host-only plan cannot run");
  const size_t need = pa_plan_workspace_bytes(plan);
  if (need > kScratchBytes)
    return pa::set_last_error(PA_ERR_INVALID_ARG, "the plan needs " + std::to_string(need) +
                                                      " bytes of workspace; the static scratch holds " +
                                                      std::to_string(kScratchBytes));
  void* ws = nullptr;
  if (need > 0) {
    const pa_status st = scratch_of(dev, &ws);
    if (st != PA_OK) return st;
  }
  return pa_forward(plan, q, kv_cache, block_table, query_start_loc, seq_lens, out, lse, ws, need ? kScratchBytes : 0,
                    stream);
}

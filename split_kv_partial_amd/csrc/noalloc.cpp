// The whole path (partial attention of every split, then the merge) for
// callers that cannot allocate device memory: code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation. The partial states
// live in a file-scope device array instead of a caller's scratch buffer.
//
// Each device that runs the library holds its own copy of the array until
// the process ends. Its address is taken once per device, with that device
// current, at the first call on it, and only that address (never the array's
// host-side name) is handed to the kernels. Every call on a device shares the
// array and leaves the last call's contents in it; calls that overlap in time
// on one device race. Nothing in it has to start at zero: every byte a call
// reads was written earlier in the same call.
#include <mutex>

#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace skv {
namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;   // 128 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device

// The current device's address of the array (looked up on first use).
skv_status device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SKV_ERR_UNSUPPORTED, "device %d: the no-allocation entry point serves devices 0-%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SKV_ERR_HIP, "hipGetSymbolAddress of the scratch array: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SKV_OK;
}

}  // namespace
}  // namespace skv

extern "C" skv_status skv_decode_attn_noalloc(const skv_attn_desc* desc, const void* q,
                                              const void* k_pages, const void* v_pages,
                                              const int32_t* page_table, const int32_t* seq_lens,
                                              const skv_plan* plan, const void* workspace, int32_t n_ext,
                                              const float* o_ext, const float* lse_ext, void* o_out,
                                              int32_t out_dtype, float* lse_out, void* stream) {
  using namespace skv;
  if (!plan) return fail(SKV_ERR_INVALID_ARG, "plan is NULL");
  const size_t need = scratch_layout(plan).total;
  if (need > kScratchBytes)
    return fail(SKV_ERR_NO_MEMORY,
                "the plan needs %zu bytes of scratch; the no-allocation entry point has %zu per device "
                "(use skv_decode_attn with a caller buffer)",
                need, kScratchBytes);
  void* ptr = nullptr;
  skv_status st = device_scratch(&ptr);
  if (st) return st;
  return decode_attn_impl(desc, q, k_pages, v_pages, page_table, seq_lens, plan, workspace, ptr,
                          kScratchBytes, n_ext, o_ext, lse_ext, o_out, out_dtype, lse_out, stream);
}

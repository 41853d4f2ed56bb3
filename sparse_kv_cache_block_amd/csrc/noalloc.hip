// noalloc.hip -- sparsekv_decode_step_noalloc: the device-pool decode step
// with its workspace in a fixed device array instead of a caller's buffer, for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops that forbid allocation).
//
// The array lives in the library's code object, one copy per GPU, for as long
// as the process runs.  Its device address differs per GPU and is looked up
// once per device with hipGetSymbolAddress; host code never passes the
// array's own name to a kernel (on the host that name is a stand-in, not a
// device address).
#include <hip/hip_runtime.h>

#include <mutex>

#include "skv_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;   // largest workspace served
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on its first
// use there (with that device current).
skv_status scratch_for_current_device(char** out) {
  int dev = 0;
  SKV_TRY_HIP(hipGetDevice(&dev), "device query");
  if (dev < 0 || dev >= kMaxDevices) return skv::fail(SKV_E_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    SKV_TRY_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "scratch address lookup");
    if (!ptr) return skv::fail(SKV_E_HIP, "scratch address lookup returned NULL");
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return SKV_OK;
}

}  // namespace

extern "C" skv_status sparsekv_decode_step_noalloc(const skv_problem* pr, const skv_step_inputs* in,
                                                   const skv_step_outputs* out, void* stream) {
  skv::Plan pl;
  SKV_TRY(skv::check_device_step(pr, in, out, &pl));
  if (pl.total_bytes > kScratchBytes)
    return skv::fail(SKV_E_WORKSPACE, "decode_step_noalloc: the problem needs %zu bytes of workspace, more than the "
                     "%zu the library holds", pl.total_bytes, kScratchBytes);
  char* ws = nullptr;
  SKV_TRY(scratch_for_current_device(&ws));
  // the arrival counters at the front must start at zero: a fill kernel
  // clears them (no memset node, so the call can be captured into a graph)
  return skv::enqueue_device_step(*pr, pl, *in, *out, ws, static_cast<hipStream_t>(stream), pl.off_scores);
}

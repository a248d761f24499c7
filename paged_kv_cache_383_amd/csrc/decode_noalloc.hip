// Scratch memory of paged_attention_decode_step_noalloc, the decode step for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The decode kernels' only scratch is the split-context workspace: fp32
// partials (m, l, acc) of each partition, written by the partition kernel and
// read by the log-sum-exp reduce within the same call (no initial contents
// needed, nothing carried between calls).  Here it is a file-scope device
// array of kStaticScratchBytes.  Every GPU the library runs on holds its own
// copy at its own address until the process ends; the array's name is only a
// host-side handle, so its device address is looked up once per device, with
// that device current, and that address is what the kernels receive.  Every
// call on one GPU shares that GPU's array: calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_internal.h"

static __device__ __align__(256) unsigned char scratch[pkv::kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];           // device address of `scratch` on each device, once looked up

}  // namespace

hipError_t pkv::static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

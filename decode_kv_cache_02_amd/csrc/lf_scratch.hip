// Static scratch memory of lf_decode_step_noalloc: the decode step's
// cross-workgroup workspace (split-K partial states, raw logits and arrival
// counters; the per-sequence score vectors, new-token norms and counters)
// taken from one file-scope device array instead of the cache's allocation.
//
// Every GPU that loads the library holds its own copy of `scratch` until the
// process ends. Host code never passes the array's name to a kernel: the name
// is a host-side stand-in, not a device address. scratch_setup() looks up the
// device address once per device (with that device current) and keeps it;
// every later use goes through scratch_ptr().
#include <hip/hip_runtime.h>

#include <mutex>

#include "lf_internal.h"

static __device__ __attribute__((aligned(256))) unsigned char scratch[lf::kScratchBytes];

namespace lf {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, null until set up

}  // namespace

hipError_t scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  // The arrival counters must start at zero; every launch that uses one
  // leaves it at zero again. Cleared synchronously here, at cache creation,
  // which is never inside a stream capture.
  e = hipMemsetAsync(p, 0, kScratchCounterBytes, nullptr);
  if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) return e;
  g_scratch_ptr[device] = p;
  return hipSuccess;
}

void* scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

}  // namespace lf

// Library-owned device scratch for the allocation-free batched decode call
// (pkv_decode_attention_noalloc): the split plan, the merge arrival counters
// and the split-K partials live in one file-scope device array, so that call
// never allocates.  Each GPU the library runs on holds its own copy of the
// array (module globals are loaded per device) until the process ends.
//
// In host code the array's name stands for a host-side shadow, not a device
// address: its device address is looked up once per device (with that device
// current) and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_internal.h"

namespace pkv {
namespace {

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace pkv

// Library-owned device scratch for pensieve_attn_fwd_noalloc: a file-scope device array that
// holds the work list and the split partials of a call, so that callers that cannot allocate
// device memory still get the whole path.  Each GPU the library runs on gets its own copy of
// the array (allocated when the code object is loaded, held until the process ends).
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address is
// looked up once per device with hipGetSymbolAddress (with that device current) and only that
// address is ever handed to kernels or copies.
#include <mutex>
#include <unordered_map>

#include "launch.h"

namespace pk {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_for_current_device(void** ptr) {
  static std::mutex mu;
  static std::unordered_map<int, void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  addr[dev] = p;
  *ptr = p;
  return hipSuccess;
}

}  // namespace pk

// Device scratch of the entry point that allocates nothing (tl_decode_step_noalloc).
//
// The buffer is one file-scope device array.  In host code its name only stands
// for the symbol, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is used
// afterwards.  Every device the library runs on holds its own copy until the
// process ends; all calls on one device share it.
#include <mutex>

#include "kernels.h"

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[device]) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device) return hipErrorInvalidDevice;   // the caller makes the device current
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_ptr[device] = p;
  return hipSuccess;
}

void* noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  return g_ptr[device];
}

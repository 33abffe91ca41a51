// step_static.hip -- the device array that holds pa_decode_step_static's partial outputs
// and LSEs, for callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// Each GPU the library runs on holds its own copy of the array from the code object's
// load until the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: the array's address on the current device is taken once per device
// with hipGetSymbolAddress, kept, and used wherever host code needs the array's memory.
#include <mutex>

#include "pa_launch.h"

namespace pa {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
char* g_address[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_address[dev] == nullptr) {   // first call on this device, which is current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_address[dev] = static_cast<char*>(p);
  }
  *out = g_address[dev];
  return hipSuccess;
}

}  // namespace pa

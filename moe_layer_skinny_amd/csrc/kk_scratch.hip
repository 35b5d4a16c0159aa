// Static device scratch for the entry point that allocates nothing (kk_layer_decode_static).
//
// `scratch` is one file-scope device array; every GPU the library runs on holds its own copy
// (at its own address) from the moment the code object is loaded on that device until the
// process ends.  In host code the array's name is only a host-side stand-in, never a device
// address: its device address is looked up with hipGetSymbolAddress once per device, with that
// device current (scratch_init, called by kk_create), and kept per device; host code passes
// that pointer, never the name, to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kk_internal.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kk::kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace kk {

hipError_t scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[device]) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device) return hipErrorInvalidDevice;  // the caller makes `device` current
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidValue;
  g_ptr[device] = p;
  return hipSuccess;
}

void* scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_ptr[device];
}

}  // namespace kk

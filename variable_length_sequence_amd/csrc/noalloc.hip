// The device scratch array behind varlen_attn_bwd_noalloc: a fixed block of
// device memory, defined in the library's code object, so that entry point
// needs no allocation of its own.  Each device the library runs on holds its
// own copy until the process ends.
//
// In host code the array's name is a host-side stand-in, not a device
// address: its address on a device is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels and copies.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "launch.h"

namespace vl {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;   // device -> address of its copy of `scratch`

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_ptr[dev] = p;
  *ptr = p;
  return hipSuccess;
}

}  // namespace vl

// Library-owned device scratch for sdit_attn_fwd_balanced_static, the entry
// point for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// One file-scope device array of kStaticScratchBytes. Each GPU that the
// library runs on holds its own copy of it, at its own address, until the
// process ends. Host code never passes the array's name to a kernel (in host
// code that name is a stand-in, not a device address): the device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and kept here; kernels receive that pointer. Every call on a GPU
// shares that GPU's array, so calls that overlap in time on one GPU race.
#include "sdit_internal.h"

#include <mutex>

namespace sdit {
namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace sdit

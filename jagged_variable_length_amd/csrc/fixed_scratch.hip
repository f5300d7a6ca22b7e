// Fixed device scratch of the backward's allocation-free entry point
// (jattn_bwd_fixed_scratch): the row statistics Di and LSE * log2(e) that the
// backward's PREP stage writes and its dK/dV and dQ stages read live here
// instead of in the caller's workspace.
//
// The array is a file-scope device variable: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code its name is only a host-side stand-in, never a device address, so the
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept; host code uses only that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace {

constexpr size_t kFixedScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kFixedScratchBytes];

std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

namespace jattn {

size_t fixed_scratch_bytes() { return kFixedScratchBytes; }

hipError_t fixed_scratch_address(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace jattn

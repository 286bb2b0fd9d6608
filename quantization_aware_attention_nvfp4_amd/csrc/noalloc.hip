// noalloc.hip - the device scratch of attn_qat_fwd_noalloc, for callers that cannot allocate
// device memory (code under stream capture, serving loops that forbid hipMalloc).
//
// The forward's workspace (K-hat rows, V-hat tiles and the variants' per-call statistics, the
// same layout attn_qat_workspace_size(0, ...) describes) lives in one file-scope device array.
// In host code the array's name is only a host-side stand-in, so its device address is looked up
// with hipGetSymbolAddress once per device (each device holds its own copy, at its own address,
// until the process ends) and that address is what the kernels receive.
#include <mutex>

#include <hip/hip_runtime.h>

#include "attnqat.h"
#include "launch.hpp"

namespace aq {
namespace {

static_assert(AQ_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch holds 256-byte aligned regions");
static __device__ __attribute__((aligned(256))) uint8_t scratch[AQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // per device: the device address of `scratch`, null until looked up

}  // namespace

hipError_t noalloc_scratch(void **out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || ((uintptr_t)p & 255)) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace aq

// noalloc.hip — the backward's scratch memory for callers that cannot allocate.
//
// fox_attn_bwd takes a caller-provided workspace for the row term and the two dc partial sums.
// fox_attn_bwd_noalloc serves callers that may not call an allocator (code under graph
// capture, tight serving loops, harnesses that forbid it): its workspace is this file's static
// device array, which every GPU the library runs on holds from module load until the process
// ends. The host never passes the array's name to a kernel: in host code that name stands for
// a host-side shadow, not a device address. The device address is looked up once per device
// with hipGetSymbolAddress, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fox_launch.h"

namespace fox {
namespace {

// The row term, dc^q, dc^k and the normalised row offset for up to 2^21 (b, h, position) rows:
// four fp32 regions of 2^21 values (32 MiB).
constexpr size_t kScratchBytes = 4 * (size_t(1) << 21) * sizeof(float);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace fox

// ipttt_chunk_delta_noalloc: the clip scales of ipttt_chunk_delta, for callers
// that cannot allocate or pass a workspace.  Its scratch (the per-token
// segment bytes, the segment table and the Gram partial sums) lives in one
// file-scope device array of IPTTT_NOALLOC_SCRATCH_BYTES, which every GPU the
// library runs on holds until the process ends.
//
// Host code never uses the array's name as an address: on the first call on a
// device, with that device current, hipGetSymbolAddress looks up the device's
// own copy, and that pointer (kept per device) is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ipttt.h"
#include "launch.h"

static __device__ __align__(256) unsigned char scratch[IPTTT_NOALLOC_SCRATCH_BYTES];

namespace ipttt {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_addr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  return hipSuccess;
}

}  // namespace ipttt

// Static scratch of libbt: device memory for the partial results of a decode step run by
// bt_decode_step_static, for callers that cannot allocate.  The array lives in the library's code
// object: every GPU the library runs on holds its own copy, from the first use until the process
// ends.  Host code never uses the array's name as a device address (on the host it only names the
// symbol); it uses the address hipGetSymbolAddress returns for the current device.
#include <mutex>

#include "bt_internal.h"

namespace bt {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace bt

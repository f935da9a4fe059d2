// scratch.hip -- the device-resident workspace of attn_paged_decode_noalloc.
//
// The split forms of the paged decode keep per-split partial outputs and
// log-sum-exps in a workspace.  For callers that cannot allocate device
// memory, this file holds one file-scope device array that serves as that
// workspace.  Every GPU the library runs on holds its own copy of the array
// until the process ends.  Host code never passes the array's name to a
// kernel: it is a host-side stand-in, not a device address.  The device
// address comes from hipGetSymbolAddress, once per device (with that device
// current), and is kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_SCRATCH_BYTES];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace attn {

// Device address of this device's copy of the scratch array, or nullptr when
// the current device cannot be queried or the symbol lookup fails.
void* decode_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_ptr[dev] = ptr;
  }
  return g_ptr[dev];
}

}  // namespace attn

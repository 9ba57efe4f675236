// The static device scratch behind ft_moe_prefill_noalloc: a file-scope device array of
// FT_PREFILL_STATIC_SCRATCH_BYTES that the code object carries, so a caller that cannot
// allocate device memory (code under HIP graph capture, a serving loop that forbids
// allocation) can still run a prefill call.  Each GPU the library runs on holds its own copy
// of the array, at its own address, until the process ends.
//
// In host code `scratch` names a host-side stand-in, not the device array: its address is
// only ever obtained through hipGetSymbolAddress, once per device with that device current,
// and that device address is what the launches receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ft_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[FT_PREFILL_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices];   // device address of `scratch` on each device, once looked up

}  // namespace

// The device address and size of the scratch on `device`, which must be the current device.
// The first call on a device looks the address up; later calls return the kept value.
extern "C" int ftk_static_scratch(int device, void** addr, size_t* bytes) {
  if (device < 0 || device >= kMaxDevices || !addr || !bytes) return (int)hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_addr[device] = p;
  }
  *addr = g_addr[device];
  *bytes = sizeof(scratch);
  return (int)hipSuccess;
}

// A fixed device array that serves as the workspace of the entry points for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  The array belongs to
// the loaded code object: every GPU the library runs on holds its own copy, at
// its own address, until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in symbol); it asks
// the runtime for the device address once per device, with that device
// current, and uses that address from then on.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace tq {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_addr[kMaxDevices] = {};  // device address of `scratch`, per device

}  // namespace

hipError_t static_scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_addr[device]) return hipSuccess;
  int current = -1;
  hipError_t e = hipGetDevice(&current);
  if (e != hipSuccess) return e;
  if (current != device) return hipErrorInvalidDevice;  // the address is looked up with `device` current
  void *ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  g_addr[device] = ptr;
  return hipSuccess;
}

void *static_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  return g_addr[device];
}

}  // namespace tq

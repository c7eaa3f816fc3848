// A fixed device workspace for the partial attention states of
// mkv_decode_static: a file-scope array that every GPU the library runs on
// holds from module load until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in symbol): the
// device address is looked up once per device with hipGetSymbolAddress and
// cached here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mkv_kernels.hpp"

namespace {

__device__ __align__(256) static uint8_t scratch[mkv::kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

namespace mkv {

hipError_t static_workspace(int device, void** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;   // the caller makes the device current
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_addr[device] = ptr;
  }
  *out = g_addr[device];
  return hipSuccess;
}

}  // namespace mkv

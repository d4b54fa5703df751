// sparse_attn_forward_noalloc: sparse_attn_forward on a library-owned device
// scratch array instead of a caller workspace, for callers that cannot call
// hipMalloc (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The array is a file-scope __device__ variable: each GPU the library runs
// on holds its own copy, allocated by the HIP runtime when the code object
// is loaded and kept until the process ends.  Host code never uses the
// variable's name as a device address (on the host it is only a stand-in):
// once per device, with that device current, hipGetSymbolAddress gives the
// device copy's address, which is kept per device and passed to the
// kernels as their workspace.
//
// Nothing in the workspace needs to start at zero (the path overwrites
// every section it reads), so the array is never cleared.  Calls that
// overlap on one GPU share that GPU's array and race: serialise them (one
// stream, or events between streams).
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "sparse_attn.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SA_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
std::vector<void*> g_scratch_ptr;  // per device; nullptr until looked up

}  // namespace

extern "C" __attribute__((visibility("hidden"))) int sparse_attn_noalloc_scratch(void** ptr) {
  if (!ptr) return SA_EINVAL;
  *ptr = nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SA_EUNSUPPORTED_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return SA_ELAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SA_OK;
}

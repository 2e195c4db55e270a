// tsa_layer_noalloc: the whole layer with every intermediate in a fixed device array of this file,
// for callers that cannot allocate at call time.  It runs tsa_layer itself on that array.
//
// The array is a file-scope __device__ variable: each GPU that loads the library's code object holds
// its own copy at its own address, for the life of the process.  In host code the array's name only
// stands in for the symbol, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tsa.h"
#include "tsa_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[TSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The scratch address on the current device, looked up on the first call there.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TSA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TSA_OK;
}

}  // namespace

extern "C" int tsa_layer_noalloc(const tsa_shape* s, const void* Q, const void* K, const void* V, const void* X,
                                 void* Y, int32_t* kLp_dev, void* stream) {
  const int st = tsa::layer_args(s, Q, K, V, X, Y, kLp_dev);
  if (st != TSA_OK) return st;
  if (tsa_layer_workspace_bytes(s) > TSA_NOALLOC_SCRATCH_BYTES) return TSA_ERR_TOO_LARGE;
  void* ws = nullptr;
  const int sa = scratch_address(&ws);
  if (sa != TSA_OK) return sa;
  return tsa_layer(s, Q, K, V, X, Y, kLp_dev, ws, TSA_NOALLOC_SCRATCH_BYTES, stream);
}

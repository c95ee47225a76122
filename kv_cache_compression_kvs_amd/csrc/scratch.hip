// Scratch memory of the allocation-free entry point (kvs_compress_block_noalloc).
//
// One file-scope device array of KVS_NOALLOC_SCRATCH_BYTES: every GPU the
// library runs on holds its own copy, from the moment this code object is
// loaded on it until the process ends.  In host code the array's name is only
// a host-side stand-in, so its device address is looked up once per device
// with hipGetSymbolAddress (that device current) and kept; kernels receive
// that address exactly as they receive a caller's workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvs_internal.h"

namespace kvs {
namespace {

__device__ __align__(256) uint8_t scratch[KVS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

int noalloc_scratch(void* stream, void** addr) {
  int dev = 0;
  if (stream) {
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess) return KVS_E_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return KVS_E_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return KVS_E_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_addr[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return KVS_E_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return KVS_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return KVS_E_HIP;
    g_addr[dev] = p;
  }
  *addr = g_addr[dev];
  return KVS_OK;
}

}  // namespace kvs

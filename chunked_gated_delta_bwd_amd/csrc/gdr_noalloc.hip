// gdr_fwd_bwd_noalloc: gdr_fwd_bwd on a workspace that the library holds in a
// file-scope device array, for callers that cannot allocate device memory.
//
// `scratch` below is an ordinary __device__ array: each GPU the library runs on
// holds its own copy (kScratchBytes) until the process ends.  Its name in host
// code is only a host-side stand-in for the symbol, so the device address of
// each GPU's copy is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is ever handed to kernels.
//
// No region of the workspace has to start at any value: every call rewrites the
// chunk and sequence tables first, and every region is written before it is
// read within the call.  Calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdr_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch` (looked up on the
// first call on the device).
gdr_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return gdr::set_error(GDR_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return gdr::set_error(GDR_EUNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return gdr::set_error(GDR_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_fwd_bwd_noalloc(const gdr_shape* shape, const gdr_inputs* in, const void* dO, const float* dht,
                               gdr_grads* grads, float* ht, void* stream) {
  size_t need = 0;
  gdr_status st = gdr_workspace_bytes(shape, &need);
  if (st != GDR_OK) return st;
  if (need > kScratchBytes)
    return gdr::set_error(GDR_EWORKSPACE,
                          "this shape needs %zu bytes of workspace; the no-allocation entry point holds %zu",
                          need, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != GDR_OK) return st;
  return gdr_fwd_bwd(shape, in, dO, dht, ws, kScratchBytes, grads, ht, stream);
}

}  // extern "C"

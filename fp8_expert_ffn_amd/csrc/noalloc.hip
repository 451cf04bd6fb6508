// Whole-layer call that allocates nothing: dmoe_forward with its workspace in
// a file-scope device array instead of a caller buffer, for callers that cannot
// call hipMalloc (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The array is a per-device global of the code object: every GPU the library
// runs on holds DMOE_NOALLOC_WS_BYTES of it until the process ends. In host
// code its name is only a host-side handle, so its device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and only
// that address is handed to kernels. Every call on one GPU uses the same
// array, which keeps the last call's contents; the kernels of dmoe_forward
// never rely on a zeroed workspace. Calls that overlap on one GPU (concurrent
// streams, or threads) race on it.
#include <mutex>

#include "dmoe_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[DMOE_NOALLOC_WS_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` per device, looked up on first use

// The device address of `scratch` on `dev`, looked up once (with `dev` current).
hipError_t scratch_on(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" dmoe_status dmoe_forward_noalloc(const dmoe_layer_desc* desc, const dmoe_layer_ptrs* ptrs,
                                            hipStream_t stream) {
  const size_t need = dmoe_forward_ws_bytes(desc);
  if (need == 0) return dmoe_forward(desc, ptrs, nullptr, 0, stream);  // reports what is wrong with desc
  if (need > (size_t)DMOE_NOALLOC_WS_BYTES)
    return dmoe::set_error(DMOE_ERR_WORKSPACE,
                           "dmoe_forward_noalloc: this layer needs %zu workspace bytes, above the %zu of the "
                           "library's fixed device array; use dmoe_forward with a caller workspace",
                           need, (size_t)DMOE_NOALLOC_WS_BYTES);
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return dmoe::set_error(DMOE_ERR_HIP, "dmoe_forward_noalloc: device of the stream: %s",
                                              hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return dmoe::set_error(DMOE_ERR_UNSUPPORTED, "dmoe_forward_noalloc: device %d beyond %d", dev, kMaxDevices);
  void* ws = nullptr;
  e = scratch_on(dev, &ws);
  if (e != hipSuccess)
    return dmoe::set_error(DMOE_ERR_HIP, "dmoe_forward_noalloc: address of the device array: %s",
                           hipGetErrorString(e));
  return dmoe_forward(desc, ptrs, ws, (size_t)DMOE_NOALLOC_WS_BYTES, stream);
}

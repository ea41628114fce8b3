// masked_attn_fwd without allocation: the forward's optional workspace (the
// key splits' partial softmax states of short query blocks, or the staged
// query-broadcast mask / bias rows) comes from a static device array that the
// library holds on every device it runs on, instead of a caller's buffer.
//
// The array's name is a host-side handle only. Its device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and only
// that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "bsm.h"
#include "bsm_internal.h"

static __device__ __align__(256) unsigned char scratch[BSM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of each device's array, once looked up

int err(int code, const char* fmt, long long a, long long b) {
  char buf[256];
  snprintf(buf, sizeof buf, fmt, a, b);
  return bsm::set_error(code, buf);
}

// The current device's scratch address (the device must be current).
int scratch_on(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      char buf[256];
      snprintf(buf, sizeof buf, "masked_attn_fwd_noalloc: scratch address on device %d: %s",
               dev, hipGetErrorString(e));
      return bsm::set_error(BSM_E_HIP, buf);
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return BSM_OK;
}

}  // namespace

extern "C" int masked_attn_fwd_noalloc(const bsm_geom* geom, const bsm_attn_args* args,
                                       hipStream_t stream) {
  if (!args) return bsm::set_error(BSM_E_ARG, "masked_attn_fwd_noalloc: args is NULL");
  if (args->workspace || args->workspace_bytes)
    return bsm::set_error(BSM_E_ARG,
                          "masked_attn_fwd_noalloc: workspace must be NULL and workspace_bytes 0 "
                          "(the call uses the library's static scratch)");
  int64_t need = 0;
  int e = attn_fwd_workspace_size(geom, args, &need);
  if (e) return e;
  if (need > BSM_NOALLOC_SCRATCH_BYTES)
    return err(BSM_E_UNSUPPORTED,
               "masked_attn_fwd_noalloc: the call needs %lld bytes of scratch; the static "
               "scratch holds %lld (use masked_attn_fwd with a workspace)",
               (long long)need, (long long)BSM_NOALLOC_SCRATCH_BYTES);
  bsm_attn_args a = *args;
  if (need > 0) {
    int dev = -1, sdev = -1;
    hipError_t he = hipGetDevice(&dev);
    if (he == hipSuccess) he = hipStreamGetDevice(stream, &sdev);
    if (he != hipSuccess)
      return bsm::set_error(BSM_E_HIP, "masked_attn_fwd_noalloc: cannot query the device");
    if (sdev != dev)
      return err(BSM_E_ARG,
                 "masked_attn_fwd_noalloc: the stream belongs to device %lld, the current "
                 "device is %lld",
                 (long long)sdev, (long long)dev);
    if (dev < 0 || dev >= kMaxDevices)
      return err(BSM_E_UNSUPPORTED, "masked_attn_fwd_noalloc: device %lld (at most %lld)",
                 (long long)dev, (long long)kMaxDevices);
    if ((e = scratch_on(dev, &a.workspace))) return e;
    a.workspace_bytes = need;
  }
  return masked_attn_fwd(geom, &a, stream);
}

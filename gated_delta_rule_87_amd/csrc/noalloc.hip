// gdr_chunk_fwd_noalloc: the chunk forward for callers that cannot allocate
// device memory.  The per-chunk quantities that gdr_chunk_fwd keeps in the
// caller's workspace go to `scratch`, a static device array that the library
// holds on every device it runs on until the process ends.
//
// In host code the name `scratch` is only a host-side stand-in for the array:
// its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and kept in scratch_ptr[]; only that address is
// passed to the kernels.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "gdr.h"
#include "kernels.hpp"

namespace {

constexpr size_t kScratchBytes = GDR_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's scratch address (looked up on its first use there).
gdr_status device_scratch(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return gdr::set_error(GDR_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return gdr::set_error(GDR_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char buf[256];
      snprintf(buf, sizeof(buf), "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return gdr::set_error(GDR_ERR_HIP, buf);
    }
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return GDR_OK;
}

}  // namespace

extern "C" gdr_status gdr_chunk_fwd_noalloc(const gdr_problem *p, const void *q, const void *k, const void *v,
                                            const void *beta, const void *log_alpha, const float *h0, void *o,
                                            float *hT, void *stream) {
  size_t need = 0;
  gdr_status s = gdr::workspace_bytes_of(p, &need);
  if (s != GDR_OK) return s;
  if (need > kScratchBytes) {
    char buf[256];
    snprintf(buf, sizeof(buf),
             "the problem needs %zu bytes of scratch; gdr_chunk_fwd_noalloc holds %zu (use gdr_chunk_fwd with a "
             "workspace)",
             need, kScratchBytes);
    return gdr::set_error(GDR_ERR_UNSUPPORTED, buf);
  }
  void *ws = nullptr;
  if (p->B > 0 && p->T > 0 && (s = device_scratch(&ws)) != GDR_OK) return s;
  // Nothing in the scratch needs clearing: the prep kernels write every byte
  // the scan kernel then reads.
  return gdr::chunk_forward(p, q, k, v, beta, log_alpha, h0, o, hT, ws, kScratchBytes, stream, true, nullptr);
}

// static_fwd.hip -- ssd_forward_fused_static: the fused forward for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).  The fused pass's
// hand-off aggregates and (packed mode) chunk table live
// in a file-scope device array instead of a caller-provided workspace; the
// kernels are those of ssd_forward(SSD_ALGO_FUSED).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "ssd.h"

namespace ssd {
// sets the thread-local message of ssd_last_error_message (api.cpp)
ssd_status api_fail(ssd_status s, const char* msg);
}

namespace {

constexpr size_t kScratchBytes = (size_t)SSD_FUSED_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// One copy per GPU, held until the process ends.  Host code never hands the
// symbol itself to a kernel (in host code it is a host-side stand-in): each
// device's address is looked up once, with that device current, and used from
// then on.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

}  // namespace

extern "C" ssd_status ssd_forward_fused_static(const ssd_problem* p, const ssd_fwd_args* a,
                                               hipStream_t stream) {
  size_t need = 0;
  const ssd_status s = ssd_workspace_size(p, SSD_ALGO_FUSED, &need);
  if (s != SSD_OK) return s;
  char buf[256];
  if (need > kScratchBytes) {
    snprintf(buf, sizeof(buf),
             "ssd_forward_fused_static: the problem needs %zu bytes of scratch, the static "
             "array holds %zu (use ssd_forward with a workspace)",
             need, kScratchBytes);
    return ssd::api_fail(SSD_ERR_WORKSPACE, buf);
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(buf, sizeof(buf), "ssd_forward_fused_static: hipGetDevice: %s",
             hipGetErrorString(e));
    return ssd::api_fail(SSD_ERR_HIP, buf);
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(buf, sizeof(buf), "ssd_forward_fused_static: device %d beyond %d", dev,
             kMaxDevices);
    return ssd::api_fail(SSD_ERR_UNSUPPORTED, buf);
  }
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> g(g_lock);
    if (!g_ptr[dev]) {
      void* q = nullptr;
      e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !q) {
        snprintf(buf, sizeof(buf), "ssd_forward_fused_static: hipGetSymbolAddress: %s",
                 hipGetErrorString(e));
        return ssd::api_fail(SSD_ERR_HIP, buf);
      }
      g_ptr[dev] = q;
    }
    ptr = g_ptr[dev];
  }
  return ssd_forward(p, SSD_ALGO_FUSED, a, ptr, kScratchBytes, stream);
}

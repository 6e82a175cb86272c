// workspace.hip -- device scratch for kernels that split one output tile over several
// workgroups (partial tiles): a library-owned stream-ordered memory pool per device, whose memory
// is kept (not released to the system) between calls, so after the first call an allocation is a
// stream-ordered reuse.  Allocation and release are ordered on the caller's stream, so calls on
// different streams never share a buffer.
#include "common.hpp"

#include <mutex>

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_pool_mu;
hipMemPool_t g_pool[kMaxDevices];

hipMemPool_t device_pool(int dev) {
  std::lock_guard<std::mutex> lk(g_pool_mu);
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  if (!g_pool[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t p = nullptr;
    if (hipMemPoolCreate(&p, &props) != hipSuccess) return nullptr;
    uint64_t keep = UINT64_MAX;
    if (hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep) != hipSuccess) {
      (void)hipMemPoolDestroy(p);
      return nullptr;
    }
    g_pool[dev] = p;
  }
  return g_pool[dev];
}

}  // namespace

int w4q_workspace_alloc(void** ptr, size_t bytes, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return W4Q_EHIP;
  hipMemPool_t pool = device_pool(dev);
  if (!pool) return W4Q_EHIP;
  return hipMallocFromPoolAsync(ptr, bytes, pool, s) == hipSuccess ? W4Q_OK : W4Q_EHIP;
}

int w4q_workspace_free(void* ptr, hipStream_t s) {
  return hipFreeAsync(ptr, s) == hipSuccess ? W4Q_OK : W4Q_EHIP;
}

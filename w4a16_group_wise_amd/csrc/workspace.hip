// workspace.hip -- device scratch for kernels that split one output tile over several
// workgroups (partial tiles).  One buffer of kWorkspaceBytes per device, allocated on first use
// and kept until the process ends.  Users are serialised: a host mutex is held from acquire to
// release, and each acquire makes the caller's stream wait for the event recorded by the
// previous release, so calls on different streams never overlap on the buffer.
#include "common.hpp"

#include <mutex>

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_buf[kMaxDevices];
hipEvent_t g_done[kMaxDevices];
bool g_used[kMaxDevices];
int g_dev = -1;  // device of the current holder

}  // namespace

int w4q_workspace_acquire(void** ptr, size_t bytes, hipStream_t s) {
  if (bytes > kWorkspaceBytes) return W4Q_EUNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W4Q_EHIP;
  g_mu.lock();
  if (!g_buf[dev]) {
    if (hipMalloc(&g_buf[dev], kWorkspaceBytes) != hipSuccess) {
      g_buf[dev] = nullptr;
      g_mu.unlock();
      return W4Q_EHIP;
    }
    if (hipEventCreateWithFlags(&g_done[dev], hipEventDisableTiming) != hipSuccess) {
      g_mu.unlock();
      return W4Q_EHIP;
    }
  }
  if (g_used[dev] && hipStreamWaitEvent(s, g_done[dev], 0) != hipSuccess) {
    g_mu.unlock();
    return W4Q_EHIP;
  }
  g_dev = dev;
  *ptr = g_buf[dev];
  return W4Q_OK;  // the mutex stays held until w4q_workspace_release
}

int w4q_workspace_release(hipStream_t s) {
  const int dev = g_dev;
  const bool ok = hipEventRecord(g_done[dev], s) == hipSuccess;
  g_used[dev] = true;
  g_mu.unlock();
  return ok ? W4Q_OK : W4Q_EHIP;
}

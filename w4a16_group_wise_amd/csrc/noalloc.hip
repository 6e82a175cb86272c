// noalloc.hip -- w4a16_gemm_dq_noalloc: the dequantizing W4A16 product for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  Its stream-K partial tiles live in `scratch`, a file-scope device array
// of kScratchBytes that every GPU the library runs on holds until the process ends; the kernels
// are those of w4a16_gemm_dq.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address is
// taken once per device with hipGetSymbolAddress (with that device current) and only that
// address is passed to kernels.  Every call on one device shares the array and leaves the
// partial tiles of its last split in it; each tile is written before the fixup reads it, so
// nothing needs clearing between calls.  Calls that overlap on one device (different streams,
// or a graph replay beside a direct call) race on the array.
#include "common.hpp"

#include <mutex>

namespace {

// the most partial tiles the fastest schedule keeps (256 workgroups x two 256x256 fp32 tiles)
constexpr size_t kScratchBytes = size_t(128) << 20;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_init_mu;               // guards the one-time address lookups only
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (nullptr: not yet)

// Device address of `scratch` on device dev, looked up once with dev current.
int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return W4Q_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_init_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return W4Q_EHIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return W4Q_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return W4Q_EHIP;
    if (e != hipSuccess || p == nullptr) return W4Q_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return W4Q_OK;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" int w4a16_gemm_dq_noalloc(const uint16_t* x, int64_t m, const uint8_t* packed,
                                     const uint16_t* scale_f16, int64_t d_out, int64_t d_in,
                                     void* y, int y_dtype, hipStream_t stream) {
  if (!x || !packed || !scale_f16 || !y || (y_dtype != 0 && y_dtype != 1)) return W4Q_EINVAL;
  if (m <= 0 || d_out <= 0 || d_in <= 0 || d_in % W4Q_GROUP != 0) return W4Q_ESHAPE;
  if (d_out > (int64_t(1) << 40) / d_in || m > (int64_t(1) << 40) / d_in ||
      m > (int64_t(1) << 40) / d_out)
    return W4Q_ESHAPE;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scale_f16, 2) ||
      !aligned(y, y_dtype == 0 ? 4 : 2))
    return W4Q_EALIGN;
  // sizes whose fastest schedule would need more scratch than the array holds are refused
  if (w4q_gemm_workspace(m, d_out, d_in, 1) > kScratchBytes) return W4Q_EUNSUPPORTED;
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return W4Q_EHIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return W4Q_EHIP;
  }
  void* ws = nullptr;
  const int rc = scratch_address(dev, &ws);
  if (rc != W4Q_OK) return rc;
  return w4q_launch_gemm(x, m, packed, scale_f16, d_out, d_in, y, y_dtype, 1, ws, kScratchBytes,
                         stream);
}

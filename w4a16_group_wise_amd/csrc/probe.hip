// probe.hip -- measured peaks that the rooflines are quoted against besides the nominal ones: a
// plain streaming read of a large buffer (HBM) and loops of independent bf16 and fp64
// matrix-core products (MFMA).  Diagnostics only; no step of the quantization path runs here.
#include "common.hpp"

namespace w4q {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;  // independent 16-byte loads in flight per lane

// Every lane reads 16-byte words at a grid stride, kReadUnroll at a time, and folds them with
// xor; the fold is stored only if it equals a value it cannot reach by chance in practice, so
// the loads stay live while almost nothing is written.  NT selects non-temporal loads.
template <bool NT>
__global__ __launch_bounds__(kReadThreads) void read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                            uint32_t* __restrict__ sink, uint32_t key) {
  uint32_t acc = 0;
  const int64_t per_iter = static_cast<int64_t>(gridDim.x) * kReadThreads * kReadUnroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kReadThreads * kReadUnroll + threadIdx.x; base < n16;
       base += per_iter) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t i = base + u * kReadThreads;
      if (i < n16)
        v[u] = NT ? __builtin_nontemporal_load(p + i) : p[i];
      else
        v[u] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == key) sink[(blockIdx.x * kReadThreads + threadIdx.x) & (W4Q_PROBE_SINK_WORDS - 1)] = acc;
}

constexpr int kMfmaChains = 16;  // independent accumulators per wavefront

__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ sink, int iters) {
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(threadIdx.x * 0.001f + e);
    b[e] = static_cast<__bf16>(e * 0.5f);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

constexpr int kF64Chains = 8;   // independent accumulators per wavefront
constexpr int kF64PerCu = 4;    // workgroups of 4 wavefronts per compute unit: 4 per SIMD

// The fold is stored only if it equals a value it cannot reach, so the products stay live.
__global__ __launch_bounds__(256) void mfma_f64_kernel(double* __restrict__ sink, int iters) {
  f64x4 acc[kF64Chains];
#pragma unroll
  for (int c = 0; c < kF64Chains; ++c) acc[c] = f64x4{0.0, 0.0, 0.0, 0.0};
  const double a = threadIdx.x * 1e-3, b = 0.5;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kF64Chains; ++c) acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[c], 0, 0, 0);
  }
  double s = 0.0;
#pragma unroll
  for (int c = 0; c < kF64Chains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == -1.0) sink[(blockIdx.x * 256 + threadIdx.x) & (W4Q_PROBE_SINK_WORDS / 2 - 1)] = s;
}

}  // namespace
}  // namespace w4q

using namespace w4q;

extern "C" {

int w4q_probe_read(const void* buf, int64_t bytes, int nontemporal, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || (nontemporal != 0 && nontemporal != 1)) return W4Q_EINVAL;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return W4Q_EALIGN;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return W4Q_EHIP;
  // 8 workgroups per compute unit: 8 wavefronts per SIMD, each with kReadUnroll loads in flight
  const int64_t n16 = bytes / 16;
  const int64_t want = (n16 + kReadThreads * kReadUnroll - 1) / (kReadThreads * kReadUnroll);
  const int64_t grid = want < static_cast<int64_t>(cus) * 8 ? want : static_cast<int64_t>(cus) * 8;
  if (nontemporal)
    hipLaunchKernelGGL(read_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(kReadThreads), 0, stream,
                       static_cast<const u32x4*>(buf), n16, sink, 0x9E3779B9u);
  else
    hipLaunchKernelGGL(read_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(kReadThreads), 0, stream,
                       static_cast<const u32x4*>(buf), n16, sink, 0x9E3779B9u);
  return w4q_launch_status();
}

int w4q_probe_mfma_bf16(float* sink, int64_t iters, double* flop, hipStream_t stream) {
  if (!sink || iters <= 0 || iters > (1 << 24)) return W4Q_EINVAL;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return W4Q_EHIP;
  // one workgroup of 4 wavefronts per compute unit: one wavefront per SIMD
  if (static_cast<int64_t>(cus) * 256 > W4Q_PROBE_SINK_WORDS) return W4Q_EUNSUPPORTED;
  hipLaunchKernelGGL(mfma_kernel, dim3(cus), dim3(256), 0, stream, sink, static_cast<int>(iters));
  if (flop) *flop = static_cast<double>(cus) * 4 * iters * kMfmaChains * (2.0 * 32 * 32 * 16);
  return w4q_launch_status();
}

int w4q_probe_mfma_f64(double* sink, int64_t iters, double* flop, hipStream_t stream) {
  if (!sink || iters <= 0 || iters > (1 << 24)) return W4Q_EINVAL;
  if (reinterpret_cast<uintptr_t>(sink) % 8 != 0) return W4Q_EALIGN;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return W4Q_EHIP;
  hipLaunchKernelGGL(mfma_f64_kernel, dim3(cus * kF64PerCu), dim3(256), 0, stream, sink, static_cast<int>(iters));
  if (flop) *flop = static_cast<double>(cus) * kF64PerCu * 4 * iters * kF64Chains * (2.0 * 16 * 16 * 4);
  return w4q_launch_status();
}

}  // extern "C"

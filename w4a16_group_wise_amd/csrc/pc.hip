// pc.hip -- the per-channel variant of export, LSQ and the W4A16 product: one scale per output
// row, the whole row as the group (model card "Opt.Gear-1B-qat-int4-per-channel-unquantized",
// intro and "Quickstart": per-channel symmetric INT4).
//
// The codes and the packed layout are those of the group-32 grid; a per-channel scale is the
// group-32 case with every group of the row on the same step.  So the row's scale is broadcast to
// d_in / 32 group scales in the caller's workspace and the group-32 kernels run unchanged: the
// codes, the forward and dW are the same operations on the same values, and the product is the
// same sum with one more rounding per group.  The step gradient of a row is the sum of its
// groups' partial sums (taken with normalisation 1), added in group order in fp64 and then
// multiplied by the row's normalisation factor.
//
// Workspace (256-byte aligned pieces): fp32 steps [d_out][G], then fp32 partial gradients or
// fp16 scales [d_out][G], then the group product's own workspace.
#include "common.hpp"

namespace w4q {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void expand_kernel(const T* __restrict__ in, int64_t rows, int64_t G,
                                                     T* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < rows * G) out[i] = in[i / G];
}

__global__ __launch_bounds__(256) void first_col_kernel(const uint16_t* __restrict__ in, int64_t rows, int64_t G,
                                                        uint16_t* __restrict__ out) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (r < rows) out[r] = in[r * G];
}

__global__ __launch_bounds__(256) void row_sum_kernel(const float* __restrict__ part, int64_t rows, int64_t G,
                                                      float gs, float* __restrict__ out) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (r >= rows) return;
  double s = 0.0;
  for (int64_t g = 0; g < G; ++g) s += static_cast<double>(part[r * G + g]);
  out[r] = static_cast<float>(static_cast<double>(gs) * s);
}

inline unsigned blocks(int64_t n) { return static_cast<unsigned>((n + 255) / 256); }
inline size_t up256(size_t b) { return (b + 255) & ~size_t(255); }

}  // namespace
}  // namespace w4q

using namespace w4q;

size_t w4q_pc_workspace(int64_t m, int64_t d_out, int64_t d_in) {
  const int64_t G = d_in / kGroup;
  const size_t a = up256(static_cast<size_t>(d_out * G) * 4);
  const size_t b = up256(static_cast<size_t>(d_out * G) * 4);
  size_t g = w4q_gemm_workspace(m, d_out, d_in, 0);
  const size_t g1 = w4q_gemm_workspace(m, d_out, d_in, 1);
  if (g1 > g) g = g1;
  return a + b + g;
}

int w4q_launch_pc(int op, const float* w, const float* scale, const float* grad, int64_t d_out, int64_t d_in,
                  float gs, float* out_w, float* out_s, float* w_hat, uint8_t* packed, uint16_t* s16_out,
                  void* ws, hipStream_t s) {
  const int64_t G = d_in / kGroup;
  const int64_t n = d_out * G;
  char* base = static_cast<char*>(ws);
  float* steps = reinterpret_cast<float*>(base);
  char* second = base + up256(static_cast<size_t>(n) * 4);
  hipLaunchKernelGGL(expand_kernel<float>, dim3(blocks(n)), dim3(256), 0, s, scale, d_out, G, steps);
  int rc = w4q_launch_status();
  if (rc != W4Q_OK) return rc;
  switch (op) {
    case 0: {  // export
      uint16_t* s16 = reinterpret_cast<uint16_t*>(second);
      if ((rc = w4q_launch_pack(w, steps, d_out, d_in, packed, s16, s)) != W4Q_OK) return rc;
      hipLaunchKernelGGL(first_col_kernel, dim3(blocks(d_out)), dim3(256), 0, s, s16, d_out, G, s16_out);
      return w4q_launch_status();
    }
    case 1:  // forward
      return w4q_launch_lsq_fwd(w, steps, d_out, d_in, w_hat, s);
    case 2: {  // backward
      float* part = reinterpret_cast<float*>(second);
      if ((rc = w4q_launch_lsq_bwd(w, steps, grad, d_out, d_in, 1.0f, out_w, part, w_hat, s)) != W4Q_OK) return rc;
      hipLaunchKernelGGL(row_sum_kernel, dim3(blocks(d_out)), dim3(256), 0, s, part, d_out, G, gs, out_s);
      return w4q_launch_status();
    }
    default:
      return W4Q_EINVAL;
  }
}

int w4q_launch_gemm_pc(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16, int64_t d_out,
                       int64_t d_in, void* y, int y_dtype, int w_mode, void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t G = d_in / kGroup;
  const int64_t n = d_out * G;
  const size_t lead = up256(static_cast<size_t>(n) * 4) * 2;
  uint16_t* sg = static_cast<uint16_t*>(ws);
  hipLaunchKernelGGL(expand_kernel<uint16_t>, dim3(blocks(n)), dim3(256), 0, s, s16, d_out, G, sg);
  const int rc = w4q_launch_status();
  if (rc != W4Q_OK) return rc;
  void* gws = static_cast<char*>(ws) + lead;
  const size_t gbytes = ws_bytes - lead;
  if (w_mode == 0 && m <= 16) return w4q_launch_gemv(x, m, packed, sg, d_out, d_in, y, y_dtype, s);
  return w4q_launch_gemm(x, m, packed, sg, d_out, d_in, y, y_dtype, w_mode, gws, gbytes, s);
}

// api.hip -- the extern "C" entry points of libw4a16q: argument checks on the host, then one
// launcher per step.  No allocation, no synchronisation, no global mutable state.
#include "common.hpp"

namespace {

constexpr int kVersion = 10000;  // 1.0.0

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// d_out x d_in weight shapes: positive, d_in a multiple of 32, element count within int64.
inline int check_wshape(int64_t d_out, int64_t d_in) {
  if (d_out <= 0 || d_in <= 0 || d_in % W4Q_GROUP != 0) return W4Q_ESHAPE;
  if (d_out > (int64_t(1) << 40) / d_in) return W4Q_ESHAPE;
  return W4Q_OK;
}

}  // namespace

extern "C" {

const char* w4q_status_string(int status) {
  switch (status) {
    case W4Q_OK: return "ok";
    case W4Q_EINVAL: return "invalid argument (null pointer, bad enum value or n_cand outside [1, 255])";
    case W4Q_ESHAPE: return "bad shape (non-positive size, d_in not a multiple of 32, ldh < d_in, d % 8 != 0 or size overflow)";
    case W4Q_EALIGN: return "misaligned pointer (tensor data must be 16-byte aligned)";
    case W4Q_EUNSUPPORTED: return "size beyond the supported range";
    case W4Q_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int w4q_version(void) { return kVersion; }

int quant_hessian(const uint16_t* x, int64_t n_tok, int64_t d, float* h, int accumulate,
                  hipStream_t stream) {
  if (!x || !h || (accumulate != 0 && accumulate != 1)) return W4Q_EINVAL;
  if (n_tok <= 0 || d <= 0 || d % 8 != 0 || d > 65536) return W4Q_ESHAPE;
  if (n_tok > (int64_t(1) << 40) / d) return W4Q_ESHAPE;
  if (!aligned(x, 16) || !aligned(h, 16)) return W4Q_EALIGN;
  return w4q_launch_hessian(x, n_tok, d, h, accumulate, stream);
}

int quant_scale_search(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
                       const float* alpha, int n_cand, float* scale, uint8_t* idx, float* obj,
                       float* obj_all, hipStream_t stream) {
  if (!w || !h || !alpha || !scale || !idx) return W4Q_EINVAL;
  if (n_cand < 1 || n_cand > W4Q_MAX_CAND) return W4Q_EINVAL;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (ldh < d_in) return W4Q_ESHAPE;
  if (!aligned(w, 16) || !aligned(h, 4) || !aligned(alpha, 4) || !aligned(scale, 4) ||
      (obj && !aligned(obj, 4)) || (obj_all && !aligned(obj_all, 4)))
    return W4Q_EALIGN;
  return w4q_launch_scale_search(w, d_out, d_in, h, ldh, alpha, n_cand, scale, idx, obj, obj_all,
                                 stream);
}

int quant_pack(const float* w, const float* scale, int64_t d_out, int64_t d_in, uint8_t* packed,
               uint16_t* scale_f16, hipStream_t stream) {
  if (!w || !scale || !packed || !scale_f16) return W4Q_EINVAL;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scale, 4) || !aligned(scale_f16, 2))
    return W4Q_EALIGN;
  return w4q_launch_pack(w, scale, d_out, d_in, packed, scale_f16, stream);
}

int lsq_fwd(const float* w, const float* scale, int64_t d_out, int64_t d_in, float* w_hat,
            hipStream_t stream) {
  if (!w || !scale || !w_hat) return W4Q_EINVAL;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (!aligned(w, 16) || !aligned(w_hat, 16) || !aligned(scale, 4)) return W4Q_EALIGN;
  return w4q_launch_lsq_fwd(w, scale, d_out, d_in, w_hat, stream);
}

int lsq_bwd(const float* w, const float* scale, const float* grad_w_hat, int64_t d_out,
            int64_t d_in, float grad_scale, float* grad_w, float* grad_scale_out, float* w_hat,
            hipStream_t stream) {
  if (!w || !scale || !grad_w_hat || !grad_w || !grad_scale_out) return W4Q_EINVAL;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (!aligned(w, 16) || !aligned(grad_w_hat, 16) || !aligned(grad_w, 16) ||
      (w_hat && !aligned(w_hat, 16)) || !aligned(scale, 4) || !aligned(grad_scale_out, 4))
    return W4Q_EALIGN;
  return w4q_launch_lsq_bwd(w, scale, grad_w_hat, d_out, d_in, grad_scale, grad_w, grad_scale_out,
                            w_hat, stream);
}

static int gemm_args(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* scale_f16,
                     int64_t d_out, int64_t d_in, void* y, int y_dtype) {
  if (!x || !packed || !scale_f16 || !y || (y_dtype != 0 && y_dtype != 1)) return W4Q_EINVAL;
  if (m <= 0) return W4Q_ESHAPE;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (m > (int64_t(1) << 40) / d_in || m > (int64_t(1) << 40) / d_out) return W4Q_ESHAPE;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scale_f16, 2) ||
      !aligned(y, y_dtype == 0 ? 4 : 2))
    return W4Q_EALIGN;
  return W4Q_OK;
}

int w4a16_gemm(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* scale_f16,
               int64_t d_out, int64_t d_in, void* y, int y_dtype, hipStream_t stream) {
  const int rc = gemm_args(x, m, packed, scale_f16, d_out, d_in, y, y_dtype);
  if (rc != W4Q_OK) return rc;
  if (m <= 16) return w4q_launch_gemv(x, m, packed, scale_f16, d_out, d_in, y, y_dtype, stream);
  return w4q_launch_gemm(x, m, packed, scale_f16, d_out, d_in, y, y_dtype, 0, stream);
}

int w4a16_gemm_dq(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* scale_f16,
                  int64_t d_out, int64_t d_in, void* y, int y_dtype, hipStream_t stream) {
  const int rc = gemm_args(x, m, packed, scale_f16, d_out, d_in, y, y_dtype);
  if (rc != W4Q_OK) return rc;
  return w4q_launch_gemm(x, m, packed, scale_f16, d_out, d_in, y, y_dtype, 1, stream);
}


int w4a16_gemv_grouped(const w4q_gemv_problem* problems, int n_problems, int y_dtype,
                       hipStream_t stream) {
  if (n_problems < 0 || (y_dtype != 0 && y_dtype != 1)) return W4Q_EINVAL;
  if (n_problems == 0) return W4Q_OK;
  if (!problems) return W4Q_EINVAL;
  for (int i = 0; i < n_problems; ++i) {
    const w4q_gemv_problem& q = problems[i];
    if (!q.x || !q.packed || !q.scale_f16 || !q.y) return W4Q_EINVAL;
    const int rc = check_wshape(q.d_out, q.d_in);
    if (rc != W4Q_OK) return rc;
    if (q.d_out > 0x7FFFFFFF || q.d_in > (int64_t(1) << 24)) return W4Q_EUNSUPPORTED;
    if (!aligned(q.x, 16) || !aligned(q.packed, 16) || !aligned(q.scale_f16, 2) ||
        !aligned(q.y, y_dtype == 0 ? 4 : 2))
      return W4Q_EALIGN;
  }
  if (!w4q_gemv_group_fits(problems, n_problems)) return W4Q_EUNSUPPORTED;
  return w4q_launch_gemv_group(problems, n_problems, y_dtype, stream);
}

}  // extern "C"

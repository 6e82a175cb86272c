// api.hip -- the extern "C" entry points of libw4a16q: argument checks on the host, then one
// launcher per step.  No allocation, no synchronisation, no global mutable state: scratch memory
// is the caller's (workspace arguments), and every call only enqueues on the caller's stream.
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
    case W4Q_ESHAPE: return "bad shape (non-positive size, d_in not a multiple of 32, ldh < d_in or not a multiple of 4, d % 8 != 0 or size overflow)";
    case W4Q_EALIGN: return "misaligned pointer (tensor data must be 16-byte aligned)";
    case W4Q_EUNSUPPORTED: return "size beyond the supported range";
    case W4Q_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int w4q_version(void) { return kVersion; }

static int hessian_args(int64_t n_tok, int64_t d) {
  if (n_tok <= 0 || d <= 0 || d % 8 != 0 || d > 65536) return W4Q_ESHAPE;
  if (n_tok > (int64_t(1) << 40) / d) return W4Q_ESHAPE;
  return W4Q_OK;
}

// scratch: NULL with 0 bytes, or 256-byte aligned memory of ws_bytes
static int ws_args(const void* ws, size_t ws_bytes) {
  if (ws == nullptr && ws_bytes != 0) return W4Q_EINVAL;
  if (ws != nullptr && !aligned(ws, 256)) return W4Q_EALIGN;
  return W4Q_OK;
}

int quant_hessian_workspace_size(int64_t n_tok, int64_t d, size_t* bytes) {
  if (!bytes) return W4Q_EINVAL;
  const int rc = hessian_args(n_tok, d);
  if (rc != W4Q_OK) return rc;
  *bytes = w4q_hessian_workspace(n_tok, d);
  return W4Q_OK;
}

int quant_hessian(const uint16_t* x, int64_t n_tok, int64_t d, float* h, int accumulate,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!x || !h || (accumulate != 0 && accumulate != 1)) return W4Q_EINVAL;
  int rc = hessian_args(n_tok, d);
  if (rc != W4Q_OK) return rc;
  if ((rc = ws_args(workspace, workspace_bytes)) != W4Q_OK) return rc;
  if (!aligned(x, 16) || !aligned(h, 16)) return W4Q_EALIGN;
  return w4q_launch_hessian(x, n_tok, d, h, accumulate, workspace, workspace_bytes, stream);
}

int quant_scale_search(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
                       const float* alpha, int n_cand, float* scale, uint8_t* idx, float* obj,
                       float* obj_all, hipStream_t stream) {
  if (!w || !h || !alpha || !scale || !idx) return W4Q_EINVAL;
  if (n_cand < 1 || n_cand > W4Q_MAX_CAND) return W4Q_EINVAL;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (ldh < d_in || ldh % 4 != 0) return W4Q_ESHAPE;
  if (!aligned(w, 16) || !aligned(h, 16) || !aligned(alpha, 4) || !aligned(scale, 4) ||
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

static bool finite_in(float v, float lo, float hi, bool lo_open) {
  if (!(v == v) || v > hi) return false;  // NaN or above
  return lo_open ? v > lo : v >= lo;
}

int lsq_adam_step(float* w, float* scale, const float* grad_w_hat, int64_t d_out, int64_t d_in,
                  float grad_scale, float* m_w, float* v_w, float* m_s, float* v_s,
                  const w4q_adam_params* hp, float* grad_scale_out, float* w_hat_next,
                  hipStream_t stream) {
  if (!w || !scale || !grad_w_hat || !m_w || !v_w || !m_s || !v_s || !hp) return W4Q_EINVAL;
  const float big = 3.0e38f;
  if (!finite_in(hp->lr_w, 0.0f, big, false) || !finite_in(hp->lr_s, 0.0f, big, false) ||
      !finite_in(hp->beta1, 0.0f, 0.99999994f, false) || !finite_in(hp->beta2, 0.0f, 0.99999994f, false) ||
      !finite_in(hp->eps, 0.0f, big, true) || !finite_in(hp->weight_decay, 0.0f, big, false) ||
      !finite_in(hp->bias_c1, 0.0f, 1.0f, true) || !finite_in(hp->bias_c2, 0.0f, 1.0f, true) ||
      !finite_in(hp->scale_min, 0.0f, big, true) || !(grad_scale == grad_scale))
    return W4Q_EINVAL;
  const int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (!aligned(w, 16) || !aligned(grad_w_hat, 16) || !aligned(m_w, 16) || !aligned(v_w, 16) ||
      (w_hat_next && !aligned(w_hat_next, 16)) || !aligned(scale, 4) || !aligned(m_s, 4) ||
      !aligned(v_s, 4) || (grad_scale_out && !aligned(grad_scale_out, 4)))
    return W4Q_EALIGN;
  return w4q_launch_lsq_adam(w, scale, grad_w_hat, d_out, d_in, grad_scale, m_w, v_w, m_s, v_s, *hp,
                             grad_scale_out, w_hat_next, stream);
}

static int gemm_shape(int64_t m, int64_t d_out, int64_t d_in);

static int gemm_args(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* scale_f16,
                     int64_t d_out, int64_t d_in, void* y, int y_dtype) {
  if (!x || !packed || !scale_f16 || !y || (y_dtype != 0 && y_dtype != 1)) return W4Q_EINVAL;
  const int rc = gemm_shape(m, d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scale_f16, 2) ||
      !aligned(y, y_dtype == 0 ? 4 : 2))
    return W4Q_EALIGN;
  return W4Q_OK;
}

static int gemm_shape(int64_t m, int64_t d_out, int64_t d_in) {
  if (m <= 0) return W4Q_ESHAPE;
  const int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (m > (int64_t(1) << 40) / d_in || m > (int64_t(1) << 40) / d_out) return W4Q_ESHAPE;
  return W4Q_OK;
}

int w4a16_gemm_workspace_size(int64_t m, int64_t d_out, int64_t d_in, size_t* bytes) {
  if (!bytes) return W4Q_EINVAL;
  const int rc = gemm_shape(m, d_out, d_in);
  if (rc != W4Q_OK) return rc;
  *bytes = w4q_gemm_workspace(m, d_out, d_in, 0);
  return W4Q_OK;
}

int w4a16_gemm_dq_workspace_size(int64_t m, int64_t d_out, int64_t d_in, size_t* bytes) {
  if (!bytes) return W4Q_EINVAL;
  const int rc = gemm_shape(m, d_out, d_in);
  if (rc != W4Q_OK) return rc;
  *bytes = w4q_gemm_workspace(m, d_out, d_in, 1);
  return W4Q_OK;
}

int w4a16_gemm(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* scale_f16,
               int64_t d_out, int64_t d_in, void* y, int y_dtype, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  int rc = gemm_args(x, m, packed, scale_f16, d_out, d_in, y, y_dtype);
  if (rc != W4Q_OK) return rc;
  if ((rc = ws_args(workspace, workspace_bytes)) != W4Q_OK) return rc;
  if (m <= 16) return w4q_launch_gemv(x, m, packed, scale_f16, d_out, d_in, y, y_dtype, stream);
  return w4q_launch_gemm(x, m, packed, scale_f16, d_out, d_in, y, y_dtype, 0, workspace,
                         workspace_bytes, stream);
}

int w4a16_gemm_dq(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* scale_f16,
                  int64_t d_out, int64_t d_in, void* y, int y_dtype, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  int rc = gemm_args(x, m, packed, scale_f16, d_out, d_in, y, y_dtype);
  if (rc != W4Q_OK) return rc;
  if ((rc = ws_args(workspace, workspace_bytes)) != W4Q_OK) return rc;
  return w4q_launch_gemm(x, m, packed, scale_f16, d_out, d_in, y, y_dtype, 1, workspace,
                         workspace_bytes, stream);
}


// ---------------------------------------------------------------- per-channel variant
static int h_args(const float* h, int64_t ldh, int64_t d_in) {
  if (ldh < d_in || ldh % 4 != 0) return W4Q_ESHAPE;
  if (!aligned(h, 16)) return W4Q_EALIGN;
  return W4Q_OK;
}

int quant_scale_search_pc(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
                          const float* alpha, int n_cand, float* scale, uint8_t* idx, float* obj,
                          float* obj_all, hipStream_t stream) {
  if (!w || !h || !alpha || !scale || !idx) return W4Q_EINVAL;
  if (n_cand < 1 || n_cand > W4Q_MAX_CAND) return W4Q_EINVAL;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (d_out > 0x7FFFFFFF) return W4Q_EUNSUPPORTED;  // one workgroup per row
  if ((rc = h_args(h, ldh, d_in)) != W4Q_OK) return rc;
  if (!aligned(w, 16) || !aligned(alpha, 4) || !aligned(scale, 4) || (obj && !aligned(obj, 4)) ||
      (obj_all && !aligned(obj_all, 4)))
    return W4Q_EALIGN;
  return w4q_launch_pc_search(w, d_out, d_in, h, ldh, alpha, n_cand, scale, idx, obj, obj_all, stream);
}

int per_channel_workspace_size(int64_t m, int64_t d_out, int64_t d_in, size_t* bytes) {
  if (!bytes) return W4Q_EINVAL;
  const int rc = gemm_shape(m, d_out, d_in);
  if (rc != W4Q_OK) return rc;
  *bytes = w4q_pc_workspace(m, d_out, d_in);
  return W4Q_OK;
}

// the per-channel workspace: present, aligned and of the size the query gives for (m, d_out, d_in)
static int pc_ws(int64_t m, int64_t d_out, int64_t d_in, const void* ws, size_t ws_bytes) {
  if (ws == nullptr) return W4Q_EINVAL;
  if (!aligned(ws, 256)) return W4Q_EALIGN;
  if (ws_bytes < w4q_pc_workspace(m, d_out, d_in)) return W4Q_EINVAL;
  return W4Q_OK;
}

int quant_pack_pc(const float* w, const float* scale, int64_t d_out, int64_t d_in, uint8_t* packed,
                  uint16_t* scale_f16, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!w || !scale || !packed || !scale_f16) return W4Q_EINVAL;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scale, 4) || !aligned(scale_f16, 2))
    return W4Q_EALIGN;
  if ((rc = pc_ws(1, d_out, d_in, workspace, workspace_bytes)) != W4Q_OK) return rc;
  return w4q_launch_pc(0, w, scale, nullptr, d_out, d_in, 0.0f, nullptr, nullptr, nullptr, packed, scale_f16,
                       workspace, stream);
}

int lsq_fwd_pc(const float* w, const float* scale, int64_t d_out, int64_t d_in, float* w_hat,
               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!w || !scale || !w_hat) return W4Q_EINVAL;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (!aligned(w, 16) || !aligned(w_hat, 16) || !aligned(scale, 4)) return W4Q_EALIGN;
  if ((rc = pc_ws(1, d_out, d_in, workspace, workspace_bytes)) != W4Q_OK) return rc;
  return w4q_launch_pc(1, w, scale, nullptr, d_out, d_in, 0.0f, nullptr, nullptr, w_hat, nullptr, nullptr,
                       workspace, stream);
}

int lsq_bwd_pc(const float* w, const float* scale, const float* grad_w_hat, int64_t d_out, int64_t d_in,
               float grad_scale, float* grad_w, float* grad_scale_out, float* w_hat, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  if (!w || !scale || !grad_w_hat || !grad_w || !grad_scale_out) return W4Q_EINVAL;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (!aligned(w, 16) || !aligned(grad_w_hat, 16) || !aligned(grad_w, 16) || (w_hat && !aligned(w_hat, 16)) ||
      !aligned(scale, 4) || !aligned(grad_scale_out, 4))
    return W4Q_EALIGN;
  if ((rc = pc_ws(1, d_out, d_in, workspace, workspace_bytes)) != W4Q_OK) return rc;
  return w4q_launch_pc(2, w, scale, grad_w_hat, d_out, d_in, grad_scale, grad_w, grad_scale_out, w_hat, nullptr,
                       nullptr, workspace, stream);
}

int w4a16_gemm_pc(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* scale_f16,
                  int64_t d_out, int64_t d_in, void* y, int y_dtype, int w_mode, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  if (w_mode != 0 && w_mode != 1) return W4Q_EINVAL;
  int rc = gemm_args(x, m, packed, scale_f16, d_out, d_in, y, y_dtype);
  if (rc != W4Q_OK) return rc;
  if ((rc = pc_ws(m, d_out, d_in, workspace, workspace_bytes)) != W4Q_OK) return rc;
  return w4q_launch_gemm_pc(x, m, packed, scale_f16, d_out, d_in, y, y_dtype, w_mode, workspace, workspace_bytes,
                            stream);
}

// ------------------------------------------------------------------- joint objective
int joint_workspace_size(int64_t d_out, int64_t d_in, size_t* bytes) {
  if (!bytes) return W4Q_EINVAL;
  const int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  *bytes = w4q_joint_workspace(d_out, d_in);
  return W4Q_OK;
}

int quant_joint_objective(const float* w, const float* scale, int64_t d_out, int64_t d_in,
                          const float* h, int64_t ldh, double* obj, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  if (!w || !scale || !h || !obj || !workspace) return W4Q_EINVAL;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if ((rc = h_args(h, ldh, d_in)) != W4Q_OK) return rc;
  if (!aligned(w, 16) || !aligned(scale, 4) || !aligned(obj, 8) || !aligned(workspace, 256)) return W4Q_EALIGN;
  return w4q_launch_joint(w, d_out, d_in, h, ldh, nullptr, 0, nullptr, const_cast<float*>(scale), 0, nullptr,
                          obj, nullptr, workspace, workspace_bytes, stream);
}

int quant_joint_refine(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
                       const float* alpha, int n_cand, uint8_t* idx, float* scale, int n_sweeps,
                       double* obj_before, double* obj_after, int32_t* sweeps, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (!w || !h || !alpha || !idx || !scale || !workspace) return W4Q_EINVAL;
  if (n_cand < 1 || n_cand > W4Q_MAX_CAND || n_sweeps < 1) return W4Q_EINVAL;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (d_out > 0x7FFFFFFF) return W4Q_EUNSUPPORTED;
  if ((rc = h_args(h, ldh, d_in)) != W4Q_OK) return rc;
  if (!aligned(w, 16) || !aligned(alpha, 4) || !aligned(scale, 4) || (obj_before && !aligned(obj_before, 8)) ||
      (obj_after && !aligned(obj_after, 8)) || (sweeps && !aligned(sweeps, 4)) || !aligned(workspace, 256))
    return W4Q_EALIGN;
  return w4q_launch_joint(w, d_out, d_in, h, ldh, alpha, n_cand, idx, scale, n_sweeps, obj_before, obj_after,
                          sweeps, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------------------ GPTQ feedback
int gptq_workspace_size(int64_t d_out, int64_t d_in, size_t* bytes) {
  if (!bytes) return W4Q_EINVAL;
  const int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (d_in > 65536) return W4Q_EUNSUPPORTED;
  *bytes = w4q_gptq_workspace(d_out, d_in);
  return W4Q_OK;
}

int quant_gptq(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
               const float* scale, float damp, float* w_hat, int32_t* info, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  if (!w || !h || !scale || !w_hat || !workspace) return W4Q_EINVAL;
  if (!(damp >= 0.0f) || damp > 3.0e38f) return W4Q_EINVAL;
  int rc = check_wshape(d_out, d_in);
  if (rc != W4Q_OK) return rc;
  if (d_in > 65536) return W4Q_EUNSUPPORTED;
  if ((rc = h_args(h, ldh, d_in)) != W4Q_OK) return rc;
  if (!aligned(w, 16) || !aligned(scale, 4) || !aligned(w_hat, 4) || (info && !aligned(info, 4)) ||
      !aligned(workspace, 256))
    return W4Q_EALIGN;
  if (workspace_bytes < w4q_gptq_workspace(d_out, d_in)) return W4Q_EINVAL;
  return w4q_launch_gptq(w, d_out, d_in, h, ldh, scale, damp, w_hat, info, workspace, stream);
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

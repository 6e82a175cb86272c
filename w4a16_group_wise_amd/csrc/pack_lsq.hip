// pack_lsq.hip -- the elementwise, HBM-bound steps: export onto the INT4 grid (quant_pack),
// the LSQ fake-quant forward (lsq_fwd), the straight-through / step-size backward (lsq_bwd), and
// the fused QAT update (lsq_adam_step: backward + Adam on weights and steps + next forward).
//
// Each thread owns 8 consecutive weights of one row (a quarter of a 32-weight group), so a
// wavefront reads and writes fully coalesced 32-byte pieces and 4 lanes share one group; the
// per-group step-size gradient is reduced across those 4 lanes (after a 2-element local sum)
// with a fixed butterfly, so results are run-to-run deterministic.
#include "common.hpp"

namespace w4q {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = 8;  // weights per thread
constexpr float kNearTie = 0.5f - 1e-5f;

// The codes of a thread's weights at step d.  The estimate comes from one reciprocal per thread
// (w * RN(1/d) is within a few units in the last place of w / d, so its nearest integer is off
// by at most one) and the exact correction step settles the code.  Steps whose reciprocal
// overflows (d below the normal range) and d <= 0 take the division per weight.
struct Coder {
  float d, inv;
  bool rcp;
  __device__ __forceinline__ explicit Coder(float step) : d(step) {
    inv = 1.0f / step;
    rcp = step > 0.0f && inv < __builtin_huge_valf();
  }
  __device__ __forceinline__ float operator()(float w) const { return rcp ? code_rcp(w, d, inv) : code_div(w, d); }
};

// Codes of 8 weights at step d as clamp(rint(w * rcp(d))).  For d in [2^-126, 2^125] the
// reciprocal is normal and w * rcp(d) is within 2e-7 relative of w / d, so that is the code
// unless w / d lies within 1e-5 of a half-integer (below 9 in magnitude; beyond, the clamp
// decides).  A wavefront with such a lane, or with a step outside that range (0 and fp32
// subnormals included), takes the exact per-weight path for all its lanes.
__device__ __forceinline__ void fast_codes(const float (&v)[8], float d, float (&c)[8]) {
  const bool ok = d >= 0x1p-126f && d <= 0x1p125f;
  const float inv = __builtin_amdgcn_rcpf(ok ? d : 1.0f);
  bool near = !ok;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = v[i] * inv;
    const float r = __builtin_rintf(t);
    near |= __builtin_fabsf(t - r) > kNearTie;
    c[i] = __builtin_fminf(__builtin_fmaxf(r, -8.0f), 7.0f);
  }
  if (__builtin_amdgcn_ballot_w64(near) != 0) {  // wave-uniform, rare
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = code_div(v[i], d);
  }
}

// Export ([card] "QAT Highlights" / "Quickstart", [blog] "Conclusion"): fp16 scale, codes on
// that scale, two's-complement nibbles with the even index in the low nibble.
__global__ __launch_bounds__(kThreads) void pack_kernel(const float* __restrict__ w,
                                                        const float* __restrict__ scale,
                                                        int64_t n8, int64_t d_in,
                                                        uint32_t* __restrict__ packed,
                                                        uint16_t* __restrict__ s16) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= n8) return;
  const int64_t e0 = t * kPer;                 // first weight (flat index)
  const int64_t grp = e0 / kGroup;             // flat group index (= row * G + g)
  const f32x4 a = *reinterpret_cast<const f32x4*>(w + e0);
  const f32x4 b = *reinterpret_cast<const f32x4*>(w + e0 + 4);
  const uint16_t hs = f32_to_f16_bits(scale[grp]);
  const float d = f16_bits_to_f32(hs);  // an fp16 value: 0, inf or normal in fp32
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  // Codes as clamp(rint(w * rcp(d))).  With w * rcp(d) within 2e-7 relative of w / d, that is the
  // code unless w / d lies within 1e-5 of a half-integer (below 9 in magnitude; beyond, the clamp
  // decides); a wavefront with such a lane takes the exact correction step for all its lanes.
  const bool pos = d > 0.0f;
  const float inv = __builtin_amdgcn_rcpf(pos ? d : 1.0f);
  float c[8];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = v[i] * inv;
    const float r = __builtin_rintf(t);
    near |= __builtin_fabsf(t - r) > kNearTie;
    c[i] = __builtin_fminf(__builtin_fmaxf(r, -8.0f), 7.0f);
  }
  if (__builtin_amdgcn_ballot_w64(near && pos) != 0) {  // wave-uniform, rare
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = code_rcp(v[i], d, inv);
  }
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = pos ? static_cast<int>(c[i]) : 0;
    word |= (static_cast<uint32_t>(q) & 0xFu) << (4 * i);
  }
  packed[t] = word;
  if ((e0 % kGroup) == 0) s16[grp] = hs;
  (void)d_in;
}

// [blog] section 3 forward: w_hat = D * code(w, D) with the fp32 learnable step D.
__global__ __launch_bounds__(kThreads) void lsq_fwd_kernel(const float* __restrict__ w,
                                                           const float* __restrict__ scale,
                                                           int64_t n8, float* __restrict__ w_hat) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= n8) return;
  const int64_t e0 = t * kPer;
  const float d = scale[e0 / kGroup];
  const f32x4 a = *reinterpret_cast<const f32x4*>(w + e0);
  const f32x4 b = *reinterpret_cast<const f32x4*>(w + e0 + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float c[8];
  fast_codes(v, d, c);
  *reinterpret_cast<f32x4*>(w_hat + e0) = f32x4{d * c[0], d * c[1], d * c[2], d * c[3]};
  *reinterpret_cast<f32x4*>(w_hat + e0 + 4) = f32x4{d * c[4], d * c[5], d * c[6], d * c[7]};
}

// [blog] section 3 backward.  m = [-8 D <= w <= 7 D] (signs from fma, exact);
// grad_w = G m;  f = q - (w / D) m;  grad_scale = gs * sum_group G f.
template <bool kFwd>
__global__ __launch_bounds__(kThreads) void lsq_bwd_kernel(const float* __restrict__ w,
                                                           const float* __restrict__ scale,
                                                           const float* __restrict__ g,
                                                           int64_t n8, float gs,
                                                           float* __restrict__ grad_w,
                                                           float* __restrict__ grad_scale,
                                                           float* __restrict__ w_hat) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool live = t < n8;
  const int64_t e0 = (live ? t : 0) * kPer;
  const float d = scale[e0 / kGroup];
  const f32x4 wa = *reinterpret_cast<const f32x4*>(w + e0);
  const f32x4 wb = *reinterpret_cast<const f32x4*>(w + e0 + 4);
  const f32x4 ga = *reinterpret_cast<const f32x4*>(g + e0);
  const f32x4 gb = *reinterpret_cast<const f32x4*>(g + e0 + 4);
  const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
  const float gv[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
  float gw[8], wh[8];
  float acc = 0.0f;
  const Coder code(d);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = code(wv[i]);
    const bool in = (__builtin_fmaf(8.0f, d, wv[i]) >= 0.0f) && (__builtin_fmaf(-7.0f, d, wv[i]) <= 0.0f);
    gw[i] = in ? gv[i] : 0.0f;
    const float f = in ? q - wv[i] / d : q;
    acc = __builtin_fmaf(gv[i], f, acc);
    wh[i] = d * q;
  }
  // 4 lanes (32 weights) per group: butterfly over lane bits 0 and 1
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  if (!live) return;
  *reinterpret_cast<f32x4*>(grad_w + e0) = f32x4{gw[0], gw[1], gw[2], gw[3]};
  *reinterpret_cast<f32x4*>(grad_w + e0 + 4) = f32x4{gw[4], gw[5], gw[6], gw[7]};
  if (kFwd) {
    *reinterpret_cast<f32x4*>(w_hat + e0) = f32x4{wh[0], wh[1], wh[2], wh[3]};
    *reinterpret_cast<f32x4*>(w_hat + e0 + 4) = f32x4{wh[4], wh[5], wh[6], wh[7]};
  }
  if ((t & 3) == 0) grad_scale[e0 / kGroup] = gs * acc;
}

// One QAT optimisation step ([blog] section 3: weights and step sizes learned jointly; [card]
// "QAT Highlights"): the gradients of lsq_bwd_kernel, then AdamW on the weights and Adam on the
// group's step (clamped at scale_min), in place; optionally the step-size gradient and the
// fake-quantised updated weights (the next forward's w_hat).  Every lane of a group computes
// the group's new step from the same reduced gradient (same bits), then the codes of its
// updated weights at that step.
template <bool kFwd>
__global__ __launch_bounds__(kThreads) void lsq_adam_kernel(float* __restrict__ w, float* __restrict__ scale,
                                                            const float* __restrict__ g, int64_t n8, float gs,
                                                            float* __restrict__ m_w, float* __restrict__ v_w,
                                                            float* __restrict__ m_s, float* __restrict__ v_s,
                                                            w4q_adam_params hp, float* __restrict__ ds_out,
                                                            float* __restrict__ w_hat) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool live = t < n8;
  const int64_t e0 = (live ? t : 0) * kPer;
  const int64_t grp = e0 / kGroup;
  const float d = scale[grp];
  float wv[8], gv[8], mv[8], vv[8];
  auto ld8 = [&](const float* p, float (&o)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p + e0);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + e0 + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  };
  auto st8 = [&](float* p, const float (&o)[8]) {
    *reinterpret_cast<f32x4*>(p + e0) = f32x4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4*>(p + e0 + 4) = f32x4{o[4], o[5], o[6], o[7]};
  };
  ld8(w, wv);
  ld8(g, gv);
  ld8(m_w, mv);
  ld8(v_w, vv);
  const float b1 = hp.beta1, b2 = hp.beta2;
  float acc = 0.0f;
  const Coder code(d);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = code(wv[i]);
    const bool in = (__builtin_fmaf(8.0f, d, wv[i]) >= 0.0f) && (__builtin_fmaf(-7.0f, d, wv[i]) <= 0.0f);
    const float gw = in ? gv[i] : 0.0f;
    const float f = in ? q - wv[i] / d : q;
    acc = __builtin_fmaf(gv[i], f, acc);
    mv[i] = b1 * mv[i] + (1.0f - b1) * gw;
    vv[i] = b2 * vv[i] + (1.0f - b2) * (gw * gw);
    const float upd = (mv[i] / hp.bias_c1) / (__builtin_sqrtf(vv[i] / hp.bias_c2) + hp.eps);
    wv[i] = wv[i] - hp.lr_w * (upd + hp.weight_decay * wv[i]);
  }
  // 4 lanes (32 weights) per group: butterfly over lane bits 0 and 1 (same sum in all four)
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  const float ds = gs * acc;
  const float ms = b1 * m_s[grp] + (1.0f - b1) * ds;
  const float vs = b2 * v_s[grp] + (1.0f - b2) * (ds * ds);
  const float dn = __builtin_fmaxf(d - hp.lr_s * ((ms / hp.bias_c1) / (__builtin_sqrtf(vs / hp.bias_c2) + hp.eps)),
                                   hp.scale_min);
  if (!live) return;
  st8(w, wv);
  st8(m_w, mv);
  st8(v_w, vv);
  if ((t & 3) == 0) {
    scale[grp] = dn;
    m_s[grp] = ms;
    v_s[grp] = vs;
    if (ds_out != nullptr) ds_out[grp] = ds;
  }
  if (kFwd) {
    const Coder next(dn);
    float wh[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wh[i] = dn * next(wv[i]);
    st8(w_hat, wh);
  }
}

inline unsigned blocks_for(int64_t n8) { return static_cast<unsigned>((n8 + kThreads - 1) / kThreads); }

}  // namespace
}  // namespace w4q

using namespace w4q;

int w4q_launch_pack(const float* w, const float* scale, int64_t d_out, int64_t d_in,
                    uint8_t* packed, uint16_t* scale_f16, hipStream_t s) {
  const int64_t n8 = d_out * d_in / kPer;
  hipLaunchKernelGGL(pack_kernel, dim3(blocks_for(n8)), dim3(kThreads), 0, s, w, scale, n8, d_in,
                     reinterpret_cast<uint32_t*>(packed), scale_f16);
  return w4q_launch_status();
}

int w4q_launch_lsq_fwd(const float* w, const float* scale, int64_t d_out, int64_t d_in,
                       float* w_hat, hipStream_t s) {
  const int64_t n8 = d_out * d_in / kPer;
  hipLaunchKernelGGL(lsq_fwd_kernel, dim3(blocks_for(n8)), dim3(kThreads), 0, s, w, scale, n8,
                     w_hat);
  return w4q_launch_status();
}

int w4q_launch_lsq_bwd(const float* w, const float* scale, const float* g, int64_t d_out,
                       int64_t d_in, float gs, float* grad_w, float* grad_scale, float* w_hat,
                       hipStream_t s) {
  const int64_t n8 = d_out * d_in / kPer;
  if (w_hat)
    hipLaunchKernelGGL(lsq_bwd_kernel<true>, dim3(blocks_for(n8)), dim3(kThreads), 0, s, w, scale,
                       g, n8, gs, grad_w, grad_scale, w_hat);
  else
    hipLaunchKernelGGL(lsq_bwd_kernel<false>, dim3(blocks_for(n8)), dim3(kThreads), 0, s, w,
                       scale, g, n8, gs, grad_w, grad_scale, w_hat);
  return w4q_launch_status();
}

int w4q_launch_lsq_adam(float* w, float* scale, const float* g, int64_t d_out, int64_t d_in, float gs,
                        float* m_w, float* v_w, float* m_s, float* v_s, const w4q_adam_params& hp,
                        float* ds_out, float* w_hat, hipStream_t s) {
  const int64_t n8 = d_out * d_in / kPer;
  if (w_hat)
    hipLaunchKernelGGL(lsq_adam_kernel<true>, dim3(blocks_for(n8)), dim3(kThreads), 0, s, w, scale, g, n8, gs,
                       m_w, v_w, m_s, v_s, hp, ds_out, w_hat);
  else
    hipLaunchKernelGGL(lsq_adam_kernel<false>, dim3(blocks_for(n8)), dim3(kThreads), 0, s, w, scale, g, n8, gs,
                       m_w, v_w, m_s, v_s, hp, ds_out, w_hat);
  return w4q_launch_status();
}

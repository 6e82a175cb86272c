// scale_search.hip -- Hessian-weighted choice of one fp16-grid scale per group of 32 weights.
//
// Method: model card "Opt.Gear-1B-qat-int4-per-channel-unquantized", "Quantization
// Configuration" (Delta* = argmin ||W X - Q_Delta(W) X||_F^2) and blog "Opt.Gear-QAT:
// Preserving On-Device Performance with QAT", section 2 (calibration activations instead of
// the max-based scale).  Read per group with the group's 32x32 diagonal block Hg of
// H = X^T X: obj_k = e_k^T Hg e_k, e_k = w - D_k code(w, D_k), D_k on the fp16 grid.
//
// Mapping (ALU-bound: ~K * 1056 flop per 137 bytes of HBM traffic): one lane scores one group;
// the 64 lanes of a wavefront hold 64 rows of the same group column g, so every element of
// Hg is wave-uniform and comes through scalar loads into SGPRs, feeding v_fma_f32 directly.
// The quadratic form uses the upper triangle (528 of 1024 entries) with 32 independent
// accumulators t_j = sum_{i<j} H_ij e_i, then obj = sum_j e_j (H_jj e_j + 2 t_j).
//
// Precision: pass 1 scores in fp32.  A group whose two best fp32 scores are within a relative
// 1e-5 (this includes exact ties and all-zero groups) is marked, and pass 2 re-scores every
// candidate of the marked groups in fp64 and takes the first minimum.  The marker is the
// index value 255, which n_cand <= 255 keeps free.
#include "common.hpp"

namespace w4q {
namespace {

constexpr int kThreads = 256;
constexpr uint8_t kMarked = 255;
constexpr float kTieRel = 1e-5f;

// Returns p unchanged but opaque to the optimiser, so loads through it are not hoisted out of
// the candidate loop (hoisting 528 H values would exhaust the registers).
__device__ __forceinline__ const float* opaque(const float* p) {
  uint64_t v = reinterpret_cast<uint64_t>(p);
  asm volatile("" : "+s"(v));
  return reinterpret_cast<const float*>(v);
}

__device__ __forceinline__ void load_group(const float* __restrict__ wp, float (&wv)[32]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(wp + 4 * i);
    wv[4 * i + 0] = v.x;
    wv[4 * i + 1] = v.y;
    wv[4 * i + 2] = v.z;
    wv[4 * i + 3] = v.w;
  }
}

__global__ __launch_bounds__(kThreads) void search_fp32_kernel(
    const float* __restrict__ w, int64_t d_out, int64_t d_in, const float* __restrict__ h,
    int64_t ldh, const float* __restrict__ alpha, int n_cand, float* __restrict__ scale,
    uint8_t* __restrict__ idx, float* __restrict__ obj, float* __restrict__ obj_all) {
  const int64_t G = d_in / kGroup;
  const int64_t g = blockIdx.y;
  const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool live = r < d_out;
  const int64_t rr = live ? r : d_out - 1;
  float wv[32];
  load_group(w + rr * d_in + g * kGroup, wv);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(wv[i]));

  const float* __restrict__ hg = h + g * kGroup * ldh + g * kGroup;  // wave-uniform
  float best = __builtin_inff(), second = __builtin_inff(), dbest = 0.0f;
  int kbest = 0;
  for (int k = 0; k < n_cand; ++k) {
    const float d = candidate(amax, alpha[k]);
    const bool zero = !(d > 0.0f);
    const float inv = __builtin_amdgcn_rcpf(zero ? 1.0f : d);
    float e[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float c = code_rcp(wv[i], d, inv);
      e[i] = zero ? wv[i] : __builtin_fmaf(-c, d, wv[i]);
    }
    const float* __restrict__ hk = opaque(hg);
    float t[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) t[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 31; ++i) {
      const float* __restrict__ hr = hk + i * ldh;
#pragma unroll
      for (int j = i + 1; j < 32; ++j) t[j] = __builtin_fmaf(hr[j], e[i], t[j]);
    }
    float o = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float u = __builtin_fmaf(2.0f, t[j], hk[j * ldh + j] * e[j]);
      o = __builtin_fmaf(e[j], u, o);
    }
    if (obj_all != nullptr && live) obj_all[(r * G + g) * n_cand + k] = o;
    if (o < best) {
      second = best;
      best = o;
      kbest = k;
      dbest = d;
    } else if (o < second) {
      second = o;
    }
  }
  if (!live) return;
  const int64_t o_ = r * G + g;
  const bool clear = (second - best) > kTieRel * best;  // false for ties, zeros and NaN
  if (clear) {
    scale[o_] = dbest;
    idx[o_] = static_cast<uint8_t>(kbest);
    if (obj != nullptr) obj[o_] = best;
  } else {
    idx[o_] = kMarked;
  }
}

// Pass 2: fp64 re-scoring of the marked groups (same grid, same codes, fp64 sums).
__global__ __launch_bounds__(kThreads) void search_fp64_kernel(
    const float* __restrict__ w, int64_t d_out, int64_t d_in, const float* __restrict__ h,
    int64_t ldh, const float* __restrict__ alpha, int n_cand, float* __restrict__ scale,
    uint8_t* __restrict__ idx, float* __restrict__ obj, float* __restrict__ obj_all) {
  const int64_t G = d_in / kGroup;
  const int64_t g = blockIdx.y;
  const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (r >= d_out) return;
  const int64_t o_ = r * G + g;
  if (idx[o_] != kMarked) return;
  float wv[32];
  load_group(w + r * d_in + g * kGroup, wv);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(wv[i]));
  const float* __restrict__ hg = h + g * kGroup * ldh + g * kGroup;
  double best = __builtin_inf();
  float dbest = 0.0f;
  int kbest = 0;
  for (int k = 0; k < n_cand; ++k) {
    const float d = candidate(amax, alpha[k]);
    const bool zero = !(d > 0.0f);
    const float inv = __builtin_amdgcn_rcpf(zero ? 1.0f : d);
    double e[32], t[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float c = zero ? 0.0f : code_rcp(wv[i], d, inv);
      e[i] = __builtin_fma(-static_cast<double>(c), static_cast<double>(d), static_cast<double>(wv[i]));
      t[i] = 0.0;
    }
    // same upper-triangle entries H[i][j], i < j, as pass 1
    const float* __restrict__ hk = opaque(hg);
#pragma unroll
    for (int i = 0; i < 31; ++i) {
      const float* __restrict__ hr = hk + i * ldh;
#pragma unroll
      for (int j = i + 1; j < 32; ++j) t[j] = __builtin_fma(static_cast<double>(hr[j]), e[i], t[j]);
    }
    double o = 0.0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const double u = __builtin_fma(2.0, t[j], static_cast<double>(hk[j * ldh + j]) * e[j]);
      o = __builtin_fma(e[j], u, o);
    }
    if (obj_all != nullptr) obj_all[o_ * n_cand + k] = static_cast<float>(o);
    if (o < best) {
      best = o;
      kbest = k;
      dbest = d;
    }
  }
  scale[o_] = dbest;
  idx[o_] = static_cast<uint8_t>(kbest);
  if (obj != nullptr) obj[o_] = static_cast<float>(best);
}

}  // namespace
}  // namespace w4q

using namespace w4q;

int w4q_launch_scale_search(const float* w, int64_t d_out, int64_t d_in, const float* h,
                            int64_t ldh, const float* alpha, int n_cand, float* scale,
                            uint8_t* idx, float* obj, float* obj_all, hipStream_t s) {
  const int64_t G = d_in / kGroup;
  if (G > 65535) return W4Q_EUNSUPPORTED;
  const dim3 grid(static_cast<unsigned>((d_out + kThreads - 1) / kThreads), static_cast<unsigned>(G));
  hipLaunchKernelGGL(search_fp32_kernel, grid, dim3(kThreads), 0, s, w, d_out, d_in, h, ldh, alpha,
                     n_cand, scale, idx, obj, obj_all);
  if (hipGetLastError() != hipSuccess) return W4Q_EHIP;
  hipLaunchKernelGGL(search_fp64_kernel, grid, dim3(kThreads), 0, s, w, d_out, d_in, h, ldh, alpha,
                     n_cand, scale, idx, obj, obj_all);
  return w4q_launch_status();
}

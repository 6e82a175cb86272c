// common.hpp -- device helpers shared by the gfx950 kernels of libw4a16q.
//
// The grid rule implemented here is the one of the symmetric INT4 quantizer with zero-point 0
// and codes in [-8, 7] (model card "Opt.Gear-1B-qat-int4-per-channel-unquantized",
// "Quantization Configuration"; blog "Opt.Gear-QAT: Preserving On-Device Performance with
// QAT", section 1): the code of w at step D is the nearest grid point for the exact real
// quotient w / D, ties to the even code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a16q.h"

namespace w4q {

constexpr int kGroup = W4Q_GROUP;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp32 -> IEEE binary16 bits, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = static_cast<_Float16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// binary16 bits -> fp32 (exact, subnormals included).
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __builtin_bit_cast(float, pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __builtin_bit_cast(float, pair & 0xFFFF0000u); }

// One correction step around an estimate c0 of the code (|c0 - code| <= 1 after clamping).
// The signs of w - (c +- 1/2) D come from single fused multiply-adds, whose rounding never
// changes a sign, so the decision is exact for any finite D > 0.  Branch-free (bitwise
// combinations of lane masks and selects).
__device__ __forceinline__ float code_correct(float w, float d, float c) {
  c = __builtin_fminf(__builtin_fmaxf(c, -8.0f), 7.0f);
  const float rh = __builtin_fmaf(-(c + 0.5f), d, w);
  const float rl = __builtin_fmaf(-(c - 0.5f), d, w);
  const float half = c * 0.5f;
  const bool odd = half != __builtin_rintf(half);
  const bool up = ((rh > 0.0f) | ((rh == 0.0f) & odd)) & (c < 7.0f);
  const bool dn = ((rl < 0.0f) | ((rl == 0.0f) & odd)) & (c > -8.0f);
  return c + (up ? 1.0f : 0.0f) - (dn ? 1.0f : 0.0f);
}

// Code of w at step d (d >= 0, finite), estimate from IEEE division.  d == 0 -> 0.
__device__ __forceinline__ float code_div(float w, float d) {
  if (!(d > 0.0f)) return 0.0f;
  return code_correct(w, d, __builtin_rintf(w / d));
}

// Code of w at step d given an approximate reciprocal inv ~ 1/d (d > 0 normal).
__device__ __forceinline__ float code_rcp(float w, float d, float inv) {
  return code_correct(w, d, __builtin_rintf(w * inv));
}

// Candidate step k of a group (fp32 in this order, then onto the fp16 grid).
__device__ __forceinline__ float candidate(float amax, float alpha) {
  const float t = alpha * amax;
  const float u = t / 7.0f;  // correctly rounded (IEEE division)
  return f16_bits_to_f32(f32_to_f16_bits(u));
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

}  // namespace w4q

// Launchers (one per source file); return a w4q_status.
int w4q_launch_hessian(const uint16_t* x, int64_t n_tok, int64_t d, float* h, int accumulate,
                       hipStream_t s);
int w4q_launch_scale_search(const float* w, int64_t d_out, int64_t d_in, const float* h,
                            int64_t ldh, const float* alpha, int n_cand, float* scale,
                            uint8_t* idx, float* obj, float* obj_all, hipStream_t s);
int w4q_launch_pack(const float* w, const float* scale, int64_t d_out, int64_t d_in,
                    uint8_t* packed, uint16_t* scale_f16, hipStream_t s);
int w4q_launch_lsq_fwd(const float* w, const float* scale, int64_t d_out, int64_t d_in,
                       float* w_hat, hipStream_t s);
int w4q_launch_lsq_bwd(const float* w, const float* scale, const float* g, int64_t d_out,
                       int64_t d_in, float gs, float* grad_w, float* grad_scale, float* w_hat,
                       hipStream_t s);
int w4q_launch_gemv(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                    int64_t d_out, int64_t d_in, void* y, int y_dtype, hipStream_t s);
int w4q_launch_gemm(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                    int64_t d_out, int64_t d_in, void* y, int y_dtype, hipStream_t s);

static inline int w4q_launch_status() {
  return hipGetLastError() == hipSuccess ? W4Q_OK : W4Q_EHIP;
}

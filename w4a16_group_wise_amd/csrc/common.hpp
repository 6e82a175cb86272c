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

typedef float f32x2 __attribute__((ext_vector_type(2)));
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

// ---------------------------------------------------------------- buffer loads to LDS
typedef int v4i32 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
constexpr uint32_t kBufferFlags = 0x00020000u;  // raw 32-bit buffer resource (gfx9 family)

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding
// (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their "no wait" maxima)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// the same, also waiting for every LDS operation of this wavefront
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes return zeros without
// touching memory.  base and bytes must be wave-uniform; readfirstlane keeps the resource in
// SGPRs (it returns int, so each half of the address is taken back as unsigned).
__device__ __forceinline__ v4i32 buffer_rsrc(const void* base, int bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  v4i32 rs;
  rs[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b)));
  rs[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b >> 32)));
  rs[2] = __builtin_amdgcn_readfirstlane(bytes);
  rs[3] = static_cast<int>(kBufferFlags);
  return rs;
}

// Buffer loads of 16 bytes per lane straight to LDS: load i fills the 1 KB of LDS at
// lds + 1024 i (lane l at + 16 l) from byte offsets vo[i].  Written as asm so that the loads may
// stay in flight across barriers (the caller waits for them with an explicit s_waitcnt); the
// blocks have no register outputs, M0 is restored, and they use only moves on scalar registers
// (no instruction that writes SCC, which the compiler may keep live across the block).
__device__ __forceinline__ void dma_x1(uint32_t lds, v4i32 rs, int v0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "buffer_load_dwordx4 %[v0], %[rs], 0 offen lds\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [m0] "s"(__builtin_amdgcn_readfirstlane(lds)), [rs] "s"(rs), [v0] "v"(v0)
      : "memory", "scc");
}
__device__ __forceinline__ void dma_x4(uint32_t lds, v4i32 rs, const int (&vo)[4]) {
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "buffer_load_dwordx4 %[v0], %[rs], 0 offen lds\n\t"
      "s_mov_b32 m0, %[m1]\n\t"
      "buffer_load_dwordx4 %[v1], %[rs], 0 offen lds\n\t"
      "s_mov_b32 m0, %[m2]\n\t"
      "buffer_load_dwordx4 %[v2], %[rs], 0 offen lds\n\t"
      "s_mov_b32 m0, %[m3]\n\t"
      "buffer_load_dwordx4 %[v3], %[rs], 0 offen lds\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [m0] "s"(l0), [m1] "s"(l0 + 1024), [m2] "s"(l0 + 2048), [m3] "s"(l0 + 3072), [rs] "s"(rs),
        [v0] "v"(vo[0]), [v1] "v"(vo[1]), [v2] "v"(vo[2]), [v3] "v"(vo[3])
      : "memory", "scc");
}
__device__ __forceinline__ void dma_x2(uint32_t lds, v4i32 rs, int v0, int v1) {
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "buffer_load_dwordx4 %[v0], %[rs], 0 offen lds\n\t"
      "s_mov_b32 m0, %[m1]\n\t"
      "buffer_load_dwordx4 %[v1], %[rs], 0 offen lds\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [m0] "s"(l0), [m1] "s"(l0 + 1024), [rs] "s"(rs), [v0] "v"(v0), [v1] "v"(v1)
      : "memory", "scc");
}
__device__ __forceinline__ void dma_x8(uint32_t lds, v4i32 rs, const int (&vo)[8]) {
  const int lo[4] = {vo[0], vo[1], vo[2], vo[3]};
  const int hi[4] = {vo[4], vo[5], vo[6], vo[7]};
  dma_x4(lds, rs, lo);
  dma_x4(lds + 4096, rs, hi);
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

}  // namespace w4q

// Launchers (one per source file); return a w4q_status.
// Scratch: the Hessian and the tiled W4A16 product split output tiles over workgroups (stream-K)
// and keep the partial tiles in scratch memory the caller passes (ws, ws_bytes); with less than
// the *_workspace size (the fastest schedule's need) they run a schedule whose partial tiles fit.
size_t w4q_hessian_workspace(int64_t n_tok, int64_t d);
size_t w4q_gemm_workspace(int64_t m, int64_t d_out, int64_t d_in, int w_mode);
int w4q_launch_hessian(const uint16_t* x, int64_t n_tok, int64_t d, float* h, int accumulate,
                       void* ws, size_t ws_bytes, hipStream_t s);
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
int w4q_launch_lsq_adam(float* w, float* scale, const float* g, int64_t d_out, int64_t d_in, float gs,
                        float* m_w, float* v_w, float* m_s, float* v_s, const w4q_adam_params& hp,
                        float* ds_out, float* w_hat, hipStream_t s);
int w4q_launch_gemv(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                    int64_t d_out, int64_t d_in, void* y, int y_dtype, hipStream_t s);
bool w4q_gemv_group_fits(const w4q_gemv_problem* probs, int n);
int w4q_launch_gemv_group(const w4q_gemv_problem* probs, int n, int y_dtype, hipStream_t s);
// w_mode: 0 = exact weights (s16 * q), 1 = weights dequantized to bf16 (RNE of s16 * q)
int w4q_launch_pc_search(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
                         const float* alpha, int n_cand, float* scale, uint8_t* idx, float* obj,
                         float* obj_all, hipStream_t s);
size_t w4q_joint_workspace(int64_t d_out, int64_t d_in);
int w4q_launch_joint(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
                     const float* alpha, int n_cand, uint8_t* idx, float* steps, int n_sweeps,
                     double* obj_before, double* obj_after, int32_t* sweeps, void* ws, size_t ws_bytes,
                     hipStream_t s);
size_t w4q_pc_workspace(int64_t m, int64_t d_out, int64_t d_in);
int w4q_launch_pc(int op, const float* w, const float* scale, const float* grad, int64_t d_out, int64_t d_in,
                  float gs, float* out_w, float* out_s, float* w_hat, uint8_t* packed, uint16_t* s16_out,
                  void* ws, hipStream_t s);
int w4q_launch_gemm_pc(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16, int64_t d_out,
                       int64_t d_in, void* y, int y_dtype, int w_mode, void* ws, size_t ws_bytes, hipStream_t s);
size_t w4q_gptq_workspace(int64_t d_out, int64_t d_in);
int w4q_launch_gptq(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh, const float* scale,
                    float damp, float* w_hat, int* info, void* ws, hipStream_t s);
int w4q_launch_gemm(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                    int64_t d_out, int64_t d_in, void* y, int y_dtype, int w_mode, void* ws,
                    size_t ws_bytes, hipStream_t s);

static inline int w4q_launch_status() {
  return hipGetLastError() == hipSuccess ? W4Q_OK : W4Q_EHIP;
}

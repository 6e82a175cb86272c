// scale_search.hip -- Hessian-weighted choice of one fp16-grid scale per group of 32 weights.
//
// Method: model card "Opt.Gear-1B-qat-int4-per-channel-unquantized", "Quantization
// Configuration" (Delta* = argmin ||W X - Q_Delta(W) X||_F^2) and blog "Opt.Gear-QAT:
// Preserving On-Device Performance with QAT", section 2 (calibration activations instead of
// the max-based scale).  Read per group with the group's 32x32 diagonal block Hg of
// H = X^T X: obj_k = e_k^T Hg e_k, e_k = w - D_k code(w, D_k), D_k on the fp16 grid.
//
// Work: K * 1056 flop per group (the symmetric quadratic form) against 137 bytes of HBM
// traffic, so the step is bound by arithmetic, not memory.  Pass 1 runs the quadratic forms
// on the fp32 matrix cores (v_mfma_f32_32x32x2_f32, full 32x32 block) with the block held in
// registers for the whole candidate loop; the mapping is described above the kernel.
//
// Codes: rint(w * rcp(D)) clamped to [-8, 7] is the exact code unless w / D lies within 1e-5
// of a half-integer (the rcp estimate is within ~2e-6 of w / D on the grid's range); when any
// lane of the wavefront hits that window, the wavefront recomputes the candidate's codes with
// the exact midpoint comparisons of code_correct.
//
// Precision: pass 1 scores in fp32.  A group whose two best fp32 scores are within a relative
// 1e-5 (this includes exact ties and all-zero groups) is marked (index value 255, which
// n_cand <= 255 keeps free), and pass 2 re-scores every candidate of each marked group in fp64,
// one candidate per lane of a wavefront, and takes the first minimum.
#include "common.hpp"

namespace w4q {
namespace {

constexpr int kThreads = 256;
constexpr uint8_t kMarked = 255;
constexpr float kTieRel = 1e-5f;
constexpr float kNear = 0.5f - 1e-5f;

// Returns p unchanged through a VGPR, opaque to the optimiser: loads through it are vector
// loads that cannot be hoisted out of the loop that produced it.
__device__ __forceinline__ const float* vopaque(const float* p) {
  uint64_t v = reinterpret_cast<uint64_t>(p);
  asm volatile("" : "+v"(v));
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

// Codes of N weights at step d (d == 0 -> all 0), as floats.
template <int N>
__device__ __forceinline__ void codes(const float (&wv)[N], float d, float (&c)[N]) {
  const bool zero = !(d > 0.0f);
  const float inv = __builtin_amdgcn_rcpf(zero ? 1.0f : d);
  bool near = false;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float t = wv[i] * inv;
    const float r = __builtin_rintf(t);
    near |= __builtin_fabsf(t - r) > kNear;
    c[i] = __builtin_fminf(__builtin_fmaxf(r, -8.0f), 7.0f);
  }
  near &= !zero;
  if (__builtin_amdgcn_ballot_w64(near) != 0) {  // wave-uniform, rare
#pragma unroll
    for (int i = 0; i < N; ++i) c[i] = code_rcp(wv[i], d, inv);
  }
  if (zero) {
#pragma unroll
    for (int i = 0; i < N; ++i) c[i] = 0.0f;
  }
}

// Pass 1 on the fp32 matrix cores.  A wavefront scores 32 rows (m = lane % 32) of one group
// column g; the two lanes of a row (h = lane / 32) each own 16 of the group's 32 positions,
// k = 8 q + 4 h + r (q, r in 0..3).  For a candidate, v_mfma_f32_32x32x2_f32 accumulates
// D = Hg * E^T over 16 steps; step s pairs position p(s, h) = 8 (s/4) + 4 h + s % 4 of every
// row, so lane (h, m) feeds e_m[p(s, h)] as the B operand and Hg[m][p(s, h)] as the A operand
// (Hg stays in 16 VGPRs for the whole candidate loop), and receives D[k][m] = (Hg e_m)[k] for
// exactly its own 16 positions k.  obj_m = sum_k e_m[k] D[k][m] is then a 16-term dot per lane
// plus one exchange with the partner lane.
__global__ __launch_bounds__(kThreads) void search_fp32_kernel(
    const float* __restrict__ w, int64_t d_out, int64_t d_in, const float* __restrict__ h,
    int64_t ldh, const float* __restrict__ alpha, int n_cand, float* __restrict__ scale,
    uint8_t* __restrict__ idx, float* __restrict__ obj, float* __restrict__ obj_all) {
  const int64_t G = d_in / kGroup;
  const int64_t g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int m = lane & 31;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / 2) + (threadIdx.x >> 6) * 32 + m;
  const bool live = r < d_out;
  const int64_t rr = live ? r : d_out - 1;

  // this lane's 16 weights and 16 entries of Hg row m, both at positions p = 8q + 4hh + (0..3)
  float wv[16], ha[16];
  const float* wp = w + rr * d_in + g * kGroup + 4 * hh;
  const float* hp = h + (g * kGroup + m) * ldh + g * kGroup + 4 * hh;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(wp + 8 * q);
    const f32x4 b = *reinterpret_cast<const f32x4*>(hp + 8 * q);
    wv[4 * q + 0] = a.x; wv[4 * q + 1] = a.y; wv[4 * q + 2] = a.z; wv[4 * q + 3] = a.w;
    ha[4 * q + 0] = b.x; ha[4 * q + 1] = b.y; ha[4 * q + 2] = b.z; ha[4 * q + 3] = b.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(wv[i]));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));

  float best = __builtin_inff(), second = __builtin_inff(), dbest = 0.0f;
  int kbest = 0;
  float a_next = alpha[0];
#pragma unroll 1
  for (int k = 0; k < n_cand; ++k) {
    const float a = a_next;
    a_next = alpha[k + 1 < n_cand ? k + 1 : k];  // scalar prefetch for the next candidate
    const float d = candidate(amax, a);
    float e[16];
    codes<16>(wv, d, e);
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = __builtin_fmaf(-e[i], d, wv[i]);
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ha[s], e[s], acc, 0, 0, 0);
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) part = __builtin_fmaf(e[i], acc[i], part);
    // both lanes of a row get the sum of the two halves (fp32 addition is commutative, so
    // both see the same bits)
    const float o = part + __shfl_xor(part, 32);
    if (obj_all != nullptr && live && hh == 0) obj_all[(r * G + g) * n_cand + k] = o;
    // running first minimum and second-smallest score (branch-free)
    const bool better = o < best;
    second = better ? best : __builtin_fminf(second, o);
    kbest = better ? k : kbest;
    dbest = better ? d : dbest;
    best = better ? o : best;
  }
  if (!live || hh != 0) return;
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

// Pass 2: fp64 re-scoring of the marked groups, one wavefront per marked group and one
// candidate per lane (same grid, same codes, fp64 sums, first minimum).
__global__ __launch_bounds__(kThreads) void search_fp64_kernel(
    const float* __restrict__ w, int64_t d_out, int64_t d_in, const float* __restrict__ h,
    int64_t ldh, const float* __restrict__ alpha, int n_cand, float* __restrict__ scale,
    uint8_t* __restrict__ idx, float* __restrict__ obj, float* __restrict__ obj_all) {
  const int64_t G = d_in / kGroup;
  const int64_t g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool marked = r < d_out && idx[r * G + g] == kMarked;
  uint64_t mask = __builtin_amdgcn_ballot_w64(marked);
  const float* __restrict__ hg = h + g * kGroup * ldh + g * kGroup;
  while (mask != 0) {
    const int src = __builtin_ctzll(mask);
    mask &= mask - 1;
    const int64_t rs = r - lane + src;  // the marked row (wave-uniform)
    const int64_t o_ = rs * G + g;
    float wv[32];
    load_group(w + rs * d_in + g * kGroup, wv);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(wv[i]));
    double best = __builtin_inf();
    int kbest = 0x7FFFFFFF;
    float dbest = 0.0f;
    for (int k0 = 0; k0 < n_cand; k0 += 64) {
      const int k = k0 + lane;
      const bool kv = k < n_cand;
      const float d = candidate(amax, alpha[kv ? k : 0]);
      float c[32];
      codes<32>(wv, d, c);  // same codes as pass 1
      double e[32];
#pragma unroll
      for (int i = 0; i < 32; ++i)
        e[i] = __builtin_fma(-static_cast<double>(c[i]), static_cast<double>(d), static_cast<double>(wv[i]));
      // o = sum_i e_i sum_j H_ij e_j over the full block, like pass 1; the outer loop stays
      // rolled and recomputes e_i from memory so no register array is indexed dynamically
      const float* hk = vopaque(hg);
      const float* wk = vopaque(w + rs * d_in + g * kGroup);
      const bool zero = !(d > 0.0f);
      const float inv = __builtin_amdgcn_rcpf(zero ? 1.0f : d);
      double o = 0.0;
#pragma unroll 1
      for (int i = 0; i < 32; ++i) {
        const float* hr = hk + i * ldh;
        double si = 0.0;
#pragma unroll
        for (int j = 0; j < 32; ++j) si = __builtin_fma(static_cast<double>(hr[j]), e[j], si);
        const float wi = wk[i];
        const float ci = zero ? 0.0f : code_rcp(wi, d, inv);
        const double ei = __builtin_fma(-static_cast<double>(ci), static_cast<double>(d), static_cast<double>(wi));
        o = __builtin_fma(ei, si, o);
      }
      if (kv) {
        if (obj_all != nullptr) obj_all[o_ * n_cand + k] = static_cast<float>(o);
        if (o < best) {  // a lane's candidates rise with k0: strict keeps the first
          best = o;
          kbest = k;
          dbest = d;
        }
      }
    }
    // wavefront argmin, ties to the lowest candidate index
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ob = __shfl_xor(best, off);
      const int ok = __shfl_xor(kbest, off);
      const float od = __shfl_xor(dbest, off);
      const bool take = (ob < best) || (ob == best && ok < kbest);
      best = take ? ob : best;
      kbest = take ? ok : kbest;
      dbest = take ? od : dbest;
    }
    if (lane == 0) {
      scale[o_] = dbest;
      idx[o_] = static_cast<uint8_t>(kbest);
      if (obj != nullptr) obj[o_] = static_cast<float>(best);
    }
  }
}

}  // namespace
}  // namespace w4q

using namespace w4q;

int w4q_launch_scale_search(const float* w, int64_t d_out, int64_t d_in, const float* h,
                            int64_t ldh, const float* alpha, int n_cand, float* scale,
                            uint8_t* idx, float* obj, float* obj_all, hipStream_t s) {
  const int64_t G = d_in / kGroup;
  if (G > 65535) return W4Q_EUNSUPPORTED;
  const dim3 grid1(static_cast<unsigned>((d_out + kThreads / 2 - 1) / (kThreads / 2)),
                   static_cast<unsigned>(G));
  hipLaunchKernelGGL(search_fp32_kernel, grid1, dim3(kThreads), 0, s, w, d_out, d_in, h, ldh, alpha,
                     n_cand, scale, idx, obj, obj_all);
  if (hipGetLastError() != hipSuccess) return W4Q_EHIP;
  const dim3 grid(static_cast<unsigned>((d_out + kThreads - 1) / kThreads), static_cast<unsigned>(G));
  hipLaunchKernelGGL(search_fp64_kernel, grid, dim3(kThreads), 0, s, w, d_out, d_in, h, ldh, alpha,
                     n_cand, scale, idx, obj, obj_all);
  return w4q_launch_status();
}

// scale_search.hip -- Hessian-weighted choice of one fp16-grid scale per group of 32 weights.
//
// Method: model card "Opt.Gear-1B-qat-int4-per-channel-unquantized", "Quantization
// Configuration" (Delta* = argmin ||W X - Q_Delta(W) X||_F^2) and blog "Opt.Gear-QAT:
// Preserving On-Device Performance with QAT", section 2 (calibration activations instead of
// the max-based scale).  Read per group with the group's 32x32 diagonal block Hg of
// H = X^T X: obj_k = e_k^T Hg e_k, e_k = w - D_k code(w, D_k), D_k on the fp16 grid.
//
// Work: K * 1056 flop per group (the symmetric quadratic form) against 137 bytes of HBM
// traffic, so the step is bound by arithmetic, not memory.  Pass 1 forms the full 32x32
// quadratic forms on the fp16 matrix cores (v_mfma_f32_32x32x16_f16) with fp32 accuracy: the
// errors and the block are each split into two fp16 parts and three part products accumulate
// in fp32 (the mapping and the error bound are described above the kernel); the block's parts
// stay in registers for the whole candidate loop.  The vector instructions (codes, splits,
// the final dot) take most of the time.
//
// Codes: rint(w * rcp(D)) clamped to [-8, 7] is the exact code unless w / D lies within 1e-5
// of a half-integer (the rcp estimate is within ~2e-6 of w / D on the grid's range); when any
// lane of the wavefront hits that window, the wavefront recomputes the candidate's codes with
// the exact midpoint comparisons of code_correct.
//
// Precision: pass 1 scores with fp32-level error (a few 2^-22 relative).  A group whose two
// best pass-1 scores are within a relative 1e-5 (this includes exact ties and all-zero groups)
// is re-scored at the end of the same workgroup: every candidate again in fp64, one candidate
// per lane, first minimum.
#include "common.hpp"

namespace w4q {
namespace {

constexpr int kThreads = 256;
constexpr float kTieRel = 1e-5f;
constexpr float kNear = 0.5f - 1e-5f;
// below this many 32-row wavefronts pass 1 runs 16 rows per wavefront
constexpr int64_t kWaves16Below = 2048;

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
template <int N, bool kZeroCodes = true>
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
  if (kZeroCodes && zero) {
#pragma unroll
    for (int i = 0; i < N; ++i) c[i] = 0.0f;
  }
}

// candidate(amax, alpha) without the IEEE division sequence: t / 7 correctly rounded as
// q0 = RN(t * RN(1/7)) followed by one fma correction with the exact remainder t - 7 q0.  Checked
// exhaustively against RN(t / 7) for every normal fp32 t (quotients below fp16's range become 0
// in the conversion either way); an infinite t (alpha * amax beyond fp32) keeps t / 7 = t.
__device__ __forceinline__ float candidate_fast(float amax, float alpha) {
  const float t = alpha * amax;
  constexpr float c = 1.0f / 7.0f;
  const float q0 = t * c;
  float q = __builtin_fmaf(__builtin_fmaf(-q0, 7.0f, t), c, q0);
  q = __builtin_fabsf(t) == __builtin_inff() ? t : q;
  return f16_bits_to_f32(f32_to_f16_bits(q));
}

// Running first minimum (score, index, step) and second-smallest score of a candidate loop,
// without branches: best = min(best, o), second = min(max(best, o), second) (a tie with the
// best makes second equal to it; NaN scores leave both unchanged), and the index and step move
// only on a strictly smaller score, so the first of equal minima is kept.
__device__ __forceinline__ void track(float o, int k, float d, float& best, float& second, int& kbest,
                                      float& dbest) {
  const bool better = o < best;
  kbest = better ? k : kbest;
  dbest = better ? d : dbest;
  second = __builtin_fminf(__builtin_fmaxf(best, o), second);
  best = __builtin_fminf(best, o);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Splits 8 fp32 values into two fp16 parts, x = hi + lo + r: hi = x rounded to fp16, lo = the
// exact fp32 difference x - hi rounded to fp16, so |lo| <= 2^-11 |x| and |r| <= 2^-22 |x| while
// the values stay in fp16's normal range (below it the parts lose at most 2^-25 absolutely).
// The values must be scaled so that |x| < 2^15.  Pairs go through v_cvt_pk_f16_f32.
__device__ __forceinline__ void split8(const float* x, f16x8& hi, f16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const float a = x[j], b = x[j + 1];
    uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
    asm volatile("" : "+v"(u));  // the parts are read back from the packed pair
    const f16x2 hp = __builtin_bit_cast(f16x2, u);
    // x - hi as one mixed-precision fma per element (exact: hi holds x's leading 11 bits)
    float ra, rb;
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(ra) : "v"(u), "v"(a));
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(rb) : "v"(u), "v"(b));
    const f16x2 lp = __builtin_convertvector((f32x2){ra, rb}, f16x2);
    hi[j] = hp[0];
    hi[j + 1] = hp[1];
    lo[j] = lp[0];
    lo[j + 1] = lp[1];
  }
}

// 2^e as a float (e in [-126, 127])
__device__ __forceinline__ float pow2(int e) { return __builtin_bit_cast(float, (e + 127) << 23); }

// Exponent that scales values whose largest magnitude is m into [2^14, 2^15): the top of
// fp16's range, so that entries far below the largest keep their bits (fp16's normal range
// ends 2^28 below the top).  Clamped to a normal power of two for m == 0 or extreme m.
__device__ __forceinline__ int scale_exp(float m) {
  const int e = __builtin_amdgcn_frexp_expf(m);  // m in [2^(e-1), 2^e)
  const int s = 15 - e;
  return s > 127 ? 127 : (s < -126 ? -126 : s);
}

// Pass 2, inside the pass-1 block: fp64 re-scoring of the rows the block marked (their two best
// pass-1 scores within kTieRel), every candidate again, one candidate per lane (same grid, same
// codes, fp64 sums, first minimum).  A block covers one group column g, so it stages Hg in LDS
// as fp64 (transposed: column j of Hg is contiguous) when any of its rows is marked, and its
// four wavefronts score each marked row together: wavefront q forms s_i = sum_j H_ij e_j and
// the partial sum of e_i s_i for the positions i = 8q .. 8q + 7, the four partials added in a
// fixed order.  e_j is recomputed from the staged weights where it is needed, so the re-scoring
// holds few registers.  Every thread of the block calls this; `marked` flags this lane's row
// (lanes below rows_per_wave own rows row0 + wavefront * rows_per_wave + lane).
__device__ __forceinline__ void rescore_marked(const float* __restrict__ w, int64_t d_in,
                                               const float* __restrict__ h, int64_t ldh,
                                               const float* __restrict__ alpha, int n_cand,
                                               float* __restrict__ scale, uint8_t* __restrict__ idx,
                                               float* __restrict__ obj, float* __restrict__ obj_all,
                                               int64_t g, int64_t row0, int rows_per_wave, bool marked) {
  static_assert(kThreads == 256, "four wavefronts share a marked row's positions");
  constexpr int kWaves = kThreads / 64;
  constexpr int kPos = kGroup / kWaves;  // positions per wavefront
  __shared__ double hs[kGroup * kGroup];
  __shared__ double part[kWaves][64];
  __shared__ uint64_t marks[kWaves];
  __shared__ float wl[kGroup];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const uint64_t mask = __builtin_amdgcn_ballot_w64(marked);
  if (!__syncthreads_or(marked)) return;  // block-uniform
  if (lane == 0) marks[wid] = mask;
  const int64_t G = d_in / kGroup;
  const float* __restrict__ hg = h + g * kGroup * ldh + g * kGroup;
  for (int t = threadIdx.x; t < kGroup * kGroup; t += kThreads)
    hs[(t % kGroup) * kGroup + t / kGroup] = static_cast<double>(hg[(t / kGroup) * ldh + t % kGroup]);
  __syncthreads();
  // every wavefront walks the same list of marked rows, so the barriers below are uniform
  for (int q = 0; q < kWaves; ++q) {
    uint64_t m = marks[q];
    while (m != 0) {
      const int src = __builtin_ctzll(m);
      m &= m - 1;
      const int64_t rs = row0 + q * rows_per_wave + src;
      const int64_t o_ = rs * G + g;
      if (threadIdx.x < kGroup) wl[threadIdx.x] = w[rs * d_in + g * kGroup + threadIdx.x];
      __syncthreads();
      float amax = __builtin_fabsf(wl[lane & (kGroup - 1)]);
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
      double best = __builtin_inf();
      int kbest = 0x7FFFFFFF;
      float dbest = 0.0f;
      for (int k0 = 0; k0 < n_cand; k0 += 64) {
        const int k = k0 + lane;
        const bool kv = k < n_cand;
        const float d = candidate_fast(amax, alpha[kv ? k : 0]);  // the step pass 1 used
        const bool zero = !(d > 0.0f);
        const float inv = __builtin_amdgcn_rcpf(zero ? 1.0f : d);
        auto err = [&](float wi) {  // e = w - code(w, d) d, exact in fp64
          const float ci = zero ? 0.0f : code_rcp(wi, d, inv);
          return __builtin_fma(-static_cast<double>(ci), static_cast<double>(d), static_cast<double>(wi));
        };
        double sv[kPos];
#pragma unroll
        for (int t = 0; t < kPos; ++t) sv[t] = 0.0;
#pragma unroll 1
        for (int j = 0; j < kGroup; ++j) {
          const double ej = err(wl[j]);
          const double* hc = hs + j * kGroup + kPos * wid;
#pragma unroll
          for (int t = 0; t < kPos; ++t) sv[t] = __builtin_fma(hc[t], ej, sv[t]);
        }
        double op = 0.0;
#pragma unroll
        for (int t = 0; t < kPos; ++t) op = __builtin_fma(err(wl[kPos * wid + t]), sv[t], op);
        part[wid][lane] = op;
        __syncthreads();
        const double o = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
        __syncthreads();  // part is rewritten by the next chunk
        if (kv) {
          if (obj_all != nullptr && wid == 0) obj_all[o_ * n_cand + k] = static_cast<float>(o);
          if (o < best) {  // a lane's candidates rise with k0: strict keeps the first
            best = o;
            kbest = k;
            dbest = d;
          }
        }
      }
      // wavefront argmin, ties to the lowest candidate index (every wavefront holds the same
      // scores; the first thread writes)
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
      if (threadIdx.x == 0) {
        scale[o_] = dbest;
        idx[o_] = static_cast<uint8_t>(kbest);
        if (obj != nullptr) obj[o_] = static_cast<float>(best);
      }
      __syncthreads();  // wl is rewritten for the next marked row
    }
  }
}

// Pass 1 on the fp16 matrix cores, fp32-accurate.  A wavefront scores 32 rows (m = lane % 32)
// of one group column g; the two lanes of a row (h = lane / 32) each own 16 of the group's 32
// positions, p = 8 q + 4 h + r (q, r in 0..3), held as element 4 q + r of the lane's arrays.
// For a candidate, D = Hg * E^T (32 positions x 32 rows) is formed by
// v_mfma_f32_32x32x16_f16 over two halves u of the reduction: in half u, reduction slot
// 8 h + t of lane (h, m) is position p with 4 q + r = 8 u + t, so the lane feeds its own
// elements 8u..8u+7 of e_m (B operand) and of Hg row m (A operand), and receives
// D[p][m] = (Hg e_m)[p] for exactly its own 16 positions.  obj_m = sum_p e_m[p] D[p][m] is a
// 16-term fp32 dot per lane plus one exchange with the partner lane.
//
// Precision: w is scaled by a power of two per row (sw) and Hg by one per block (sh), both
// exactly, so that their largest magnitudes sit in [2^14, 2^15); the scaled error
// e = sw w - code * (sw D) is exact in fp32 and |e| <= |sw w| (a code never overshoots w by
// more than D / 2 <= |w|, and a clamped or zero code only shrinks w), so nothing overflows fp16.
// e and Hg are each split into two fp16 parts (relative residual <= 2^-22 in fp16's normal
// range), and D accumulates hi*lo, lo*hi, then hi*hi in fp32 (products of fp16 values are
// exact; the dropped lo*lo term is <= 2^-22 relative), so the score carries an error of a few
// 2^-22 of the form's magnitude before the exact rescale by 2^-(2 log2 sw + log2 sh).  The
// headroom matters when the channel scales of X spread widely: the block's small entries then
// lie many binades below its largest one and still need their full 22 bits.
template <bool kAll>
__global__ __launch_bounds__(kThreads, 5) void search_split_kernel(
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
  float amax = 0.0f, hmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax = __builtin_fmaxf(amax, __builtin_fabsf(wv[i]));
    hmax = __builtin_fmaxf(hmax, __builtin_fabsf(ha[i]));
  }
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) hmax = __builtin_fmaxf(hmax, __shfl_xor(hmax, off));

  // exact power-of-two scalings, then the two fp16 parts of the block (A operands)
  const int ew = scale_exp(amax), eh = scale_exp(hmax);
  const float sw = pow2(ew), sh = pow2(eh);
  const int unscale = -(2 * ew + eh);  // obj = score * 2^unscale
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    wv[i] *= sw;
    ha[i] *= sh;
  }
  f16x8 hhi[2], hlo[2];
  split8(ha, hhi[0], hlo[0]);
  split8(ha + 8, hhi[1], hlo[1]);

  float best = __builtin_inff(), second = __builtin_inff(), dbest = 0.0f;
  int kbest = 0;
  float d_next = candidate_fast(amax, alpha[0]);
#pragma unroll 1
  for (int k = 0; k < n_cand; ++k) {
    const float d = d_next;
    // the next candidate's step, off this candidate's dependency chain
    d_next = candidate_fast(amax, alpha[k + 1 < n_cand ? k + 1 : k]);
    const float ds = d * sw;  // exact; the codes of sw w at ds are those of w at d
    float e[16];
    // at a zero step the error is w whatever the codes are (w - c * 0), so the codes need not
    // be cleared for it
    codes<16, false>(wv, ds, e);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      e[i] = __builtin_fmaf(-e[i], ds, wv[i]);
      asm volatile("" : "+v"(e[i]));  // e is formed once in fp32, then split
    }
    f16x8 ehi[2], elo[2];
    split8(e, ehi[0], elo[0]);
    split8(e + 8, ehi[1], elo[1]);
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(hhi[u], elo[u], acc, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 2; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(hlo[u], ehi[u], acc, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 2; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(hhi[u], ehi[u], acc, 0, 0, 0);
    float p0 = 0.0f, p1 = 0.0f;  // two chains: even and odd positions of the lane
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      p0 = __builtin_fmaf(e[i], acc[i], p0);
      p1 = __builtin_fmaf(e[i + 1], acc[i + 1], p1);
    }
    const float part = p0 + p1;
    // both lanes of a row get lo-half + hi-half of the two partial dots (same bits in both)
    const auto pr = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, part),
                                                     __builtin_bit_cast(uint32_t, part), false, false);
    const uint32_t u0 = pr[0], u1 = pr[1];
    const float o = __builtin_ldexpf(__builtin_bit_cast(float, u0) + __builtin_bit_cast(float, u1), unscale);
    if (kAll && live && hh == 0) obj_all[(r * G + g) * n_cand + k] = o;
    track(o, k, d, best, second, kbest, dbest);
  }
  const bool clear = (second - best) > kTieRel * best;  // false for ties, zeros and NaN
  if (live && hh == 0 && clear) {
    const int64_t o_ = r * G + g;
    scale[o_] = dbest;
    idx[o_] = static_cast<uint8_t>(kbest);
    if (obj != nullptr) obj[o_] = best;
  }
  rescore_marked(w, d_in, h, ldh, alpha, n_cand, scale, idx, obj, obj_all, g,
                 (int64_t)blockIdx.x * (kThreads / 2), 32, live && hh == 0 && !clear);
}

// Pass 1 for small grids: 16 rows per wavefront (twice the wavefronts of the kernel above, so
// short problems still fill the SIMDs).  Lane (q, j) = (lane / 16, lane % 16) owns positions
// p = 8 q + e (e = 0..7) of row j.  v_mfma_f32_32x32x16_f16 is replaced by pairs of
// v_mfma_f32_16x16x32_f16: product u (0, 1) has output rows i = 0..15 standing for positions
// 8 (i / 4) + 4 u + i % 4 and the reduction slot 8 q + e standing for position 8 q + e, so the
// lane feeds its own 8 errors as the B operand and Hg[8 (i / 4) + 4 u + i % 4][8 q + e] (i = the
// lane's j) as the A operand, and receives D[p][j] for exactly its own positions
// p = 8 q + 4 u + r (r = 0..3).  Scaling, splitting and accumulation order as above.
template <bool kAll>
__global__ __launch_bounds__(kThreads) void search_split16_kernel(
    const float* __restrict__ w, int64_t d_out, int64_t d_in, const float* __restrict__ h,
    int64_t ldh, const float* __restrict__ alpha, int n_cand, float* __restrict__ scale,
    uint8_t* __restrict__ idx, float* __restrict__ obj, float* __restrict__ obj_all) {
  const int64_t G = d_in / kGroup;
  const int64_t g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int j = lane & 15;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / 4) + (threadIdx.x >> 6) * 16 + j;
  const bool live = r < d_out;
  const int64_t rr = live ? r : d_out - 1;

  // this lane's 8 weights (positions 8q .. 8q+7) and, for u = 0, 1, the same 8 columns of Hg
  // row 8 (j / 4) + 4 u + j % 4
  float wv[8], ha[2][8];
  {
    const float* wp = w + rr * d_in + g * kGroup + 8 * q;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(wp);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(wp + 4);
    wv[0] = a0.x; wv[1] = a0.y; wv[2] = a0.z; wv[3] = a0.w;
    wv[4] = a1.x; wv[5] = a1.y; wv[6] = a1.z; wv[7] = a1.w;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int prow = 8 * (j >> 2) + 4 * u + (j & 3);
      const float* hp = h + (g * kGroup + prow) * ldh + g * kGroup + 8 * q;
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(hp);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(hp + 4);
      ha[u][0] = b0.x; ha[u][1] = b0.y; ha[u][2] = b0.z; ha[u][3] = b0.w;
      ha[u][4] = b1.x; ha[u][5] = b1.y; ha[u][6] = b1.z; ha[u][7] = b1.w;
    }
  }
  float amax = 0.0f, hmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    amax = __builtin_fmaxf(amax, __builtin_fabsf(wv[i]));
    hmax = __builtin_fmaxf(hmax, __builtin_fmaxf(__builtin_fabsf(ha[0][i]), __builtin_fabsf(ha[1][i])));
  }
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) hmax = __builtin_fmaxf(hmax, __shfl_xor(hmax, off));

  const int ew = scale_exp(amax), eh = scale_exp(hmax);
  const float sw = pow2(ew), sh = pow2(eh);
  const int unscale = -(2 * ew + eh);  // obj = score * 2^unscale
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    wv[i] *= sw;
    ha[0][i] *= sh;
    ha[1][i] *= sh;
  }
  f16x8 hhi[2], hlo[2];
  split8(ha[0], hhi[0], hlo[0]);
  split8(ha[1], hhi[1], hlo[1]);

  float best = __builtin_inff(), second = __builtin_inff(), dbest = 0.0f;
  int kbest = 0;
  float d_next = candidate_fast(amax, alpha[0]);
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 1
  for (int k = 0; k < n_cand; ++k) {
    const float d = d_next;
    // the next candidate's step, off this candidate's dependency chain
    d_next = candidate_fast(amax, alpha[k + 1 < n_cand ? k + 1 : k]);
    const float ds = d * sw;  // exact; the codes of sw w at ds are those of w at d
    float e[8];
    codes<8, false>(wv, ds, e);  // at a zero step the error is w whatever the codes are
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e[i] = __builtin_fmaf(-e[i], ds, wv[i]);
      asm volatile("" : "+v"(e[i]));  // e is formed once in fp32, then split
    }
    f16x8 ehi, elo;
    split8(e, ehi, elo);
    f32x4 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hhi[u], elo, zero4, 0, 0, 0);
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hlo[u], ehi, acc[u], 0, 0, 0);
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hhi[u], ehi, acc[u], 0, 0, 0);
    }
    float p0 = 0.0f, p1 = 0.0f;  // two chains: the two products
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0 = __builtin_fmaf(e[i], acc[0][i], p0);
      p1 = __builtin_fmaf(e[4 + i], acc[1][i], p1);
    }
    const float part = p0 + p1;
    // the four lanes of a row add their partial dots pairwise: (q0 + q1) + (q2 + q3) in all of
    // them (same bits in each)
    const auto s1 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, part),
                                                     __builtin_bit_cast(uint32_t, part), false, false);
    const uint32_t a0 = s1[0], a1 = s1[1];
    const float half = __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
    const auto s2 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, half),
                                                     __builtin_bit_cast(uint32_t, half), false, false);
    const uint32_t b0 = s2[0], b1 = s2[1];
    const float o = __builtin_ldexpf(__builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1), unscale);
    if (kAll && live && q == 0) obj_all[(r * G + g) * n_cand + k] = o;
    track(o, k, d, best, second, kbest, dbest);
  }
  const bool clear = (second - best) > kTieRel * best;  // false for ties, zeros and NaN
  if (live && q == 0 && clear) {
    const int64_t o_ = r * G + g;
    scale[o_] = dbest;
    idx[o_] = static_cast<uint8_t>(kbest);
    if (obj != nullptr) obj[o_] = best;
  }
  rescore_marked(w, d_in, h, ldh, alpha, n_cand, scale, idx, obj, obj_all, g,
                 (int64_t)blockIdx.x * (kThreads / 4), 16, live && q == 0 && !clear);
}

}  // namespace
}  // namespace w4q

using namespace w4q;

int w4q_launch_scale_search(const float* w, int64_t d_out, int64_t d_in, const float* h,
                            int64_t ldh, const float* alpha, int n_cand, float* scale,
                            uint8_t* idx, float* obj, float* obj_all, hipStream_t s) {
  const int64_t G = d_in / kGroup;
  if (G > 65535) return W4Q_EUNSUPPORTED;
  // 32 rows per wavefront, or 16 when that leaves too few wavefronts to fill the SIMDs
  const int64_t waves32 = (d_out + 31) / 32 * G;
  if (waves32 >= kWaves16Below) {
    const dim3 grid1(static_cast<unsigned>((d_out + kThreads / 2 - 1) / (kThreads / 2)),
                     static_cast<unsigned>(G));
    if (obj_all != nullptr)
      hipLaunchKernelGGL(search_split_kernel<true>, grid1, dim3(kThreads), 0, s, w, d_out, d_in, h, ldh,
                         alpha, n_cand, scale, idx, obj, obj_all);
    else
      hipLaunchKernelGGL(search_split_kernel<false>, grid1, dim3(kThreads), 0, s, w, d_out, d_in, h, ldh,
                         alpha, n_cand, scale, idx, obj, obj_all);
  } else {
    const dim3 grid1(static_cast<unsigned>((d_out + kThreads / 4 - 1) / (kThreads / 4)),
                     static_cast<unsigned>(G));
    if (obj_all != nullptr)
      hipLaunchKernelGGL(search_split16_kernel<true>, grid1, dim3(kThreads), 0, s, w, d_out, d_in, h, ldh,
                         alpha, n_cand, scale, idx, obj, obj_all);
    else
      hipLaunchKernelGGL(search_split16_kernel<false>, grid1, dim3(kThreads), 0, s, w, d_out, d_in, h, ldh,
                         alpha, n_cand, scale, idx, obj, obj_all);
  }
  return w4q_launch_status();
}

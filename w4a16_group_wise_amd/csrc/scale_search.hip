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
// Precision: pass 1 scores with fp32-level error and bounds it: with each score o it forms
// B = |e|^T |Hg| |e| on the matrix cores and takes r = 2^-18 B as the score's radius (the
// exact objective lies within o +- r).  A group's choice is kept when the best candidate's
// interval lies below every other candidate's interval and its radius is below 9e-6 of its
// score; otherwise (near-ties, exact ties, all-zero groups, ill-conditioned blocks where the
// form cancels) the candidates whose intervals reach below the best one are re-scored in fp64
// at the end of the same workgroup, and the first minimum among them is taken.
#include "common.hpp"

#include <utility>

// every multiply and add below rounds as written (no contraction into fused operations): the
// radii and interval tests are evaluated exactly as the error analysis states them
#pragma clang fp contract(off)

namespace w4q {
namespace {

constexpr int kThreads = 256;
constexpr float kNear = 0.5f - 1e-5f;
// below this many 32-row wavefronts pass 1 runs 16 rows per wavefront
constexpr int64_t kWaves16Below = 2048;

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
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(near) != 0, 0)) {  // wave-uniform, rare
    // (the empty asm keeps this a branch: as selects, the exact rule would run every time)
    asm volatile("");
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

// |x| of eight fp16 values (sign bits cleared)
__device__ __forceinline__ f16x8 abs8(f16x8 x) {
  u32x4 u = __builtin_bit_cast(u32x4, x);
  u &= 0x7FFF7FFFu;
  return __builtin_bit_cast(f16x8, u);
}

// a + (the same quantity in the lane 32 apart): both lanes of a row get lo-half + hi-half of the
// two partial dots (the same bits in both)
__device__ __forceinline__ float pair_sum32(float part) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, part),
                                                   __builtin_bit_cast(uint32_t, part), false, false);
  const uint32_t u0 = pr[0], u1 = pr[1];
  return __builtin_bit_cast(float, u0) + __builtin_bit_cast(float, u1);
}

// sum over the four lanes 16 apart, added pairwise: (q0 + q1) + (q2 + q3) in all of them (same
// bits in each)
__device__ __forceinline__ float quad_sum(float part) {
  const auto s1 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, part),
                                                   __builtin_bit_cast(uint32_t, part), false, false);
  const uint32_t a0 = s1[0], a1 = s1[1];
  return pair_sum32(__builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1));
}

// Error radius of a pass-1 score.  Pass 1 evaluates e^T Hg e from fp16 parts (two per value,
// relative residual <= 2^-22), dropping the lo*lo product, with fp32 accumulation in six
// matrix-core products of 16 terms each and a final 16-term fp32 dot.  Every one of these
// errors is a small multiple of 2^-24 or 2^-22 times a sum of |e_i| |H_ij| |e_j| terms, so
// the score's error is at most a constant times B = |e|^T |Hg| |e| (with one rounding per
// matrix-core product the constant is about 7 * 2^-22).  Pass 1 also evaluates B, from the hi
// parts of |Hg| and |e| on the matrix cores (accurate to about 2^-10, ample for a bound), and
// takes kRad * B as the radius of the score: the exact objective lies in [o - r, o + r].
// kRad = 2^-18 = 16 * 2^-22 is three times the largest error measured against the fp64 oracle
// (5.3 * 2^-22 B, over every candidate of iid, lognormal(0, 2.5) and correlated calibration
// data), and above the model's constant.
constexpr float kRad = 1.0f / 262144.0f;  // 2^-18
// A pass-1 objective is returned only if its radius is below this fraction of it (the
// objective is then within 1e-5 relative of the exact value, fp32 output rounding included).
constexpr float kObjRel = 9e-6f;

// Running state of a candidate loop over one row (all values in the row's scaled units):
// the first minimum (best, kbest, dbest) with its radius, and the three smallest lower ends
// o - r of the candidates' intervals (the two smallest with their indices).
struct Track {
  float best = __builtin_inff(), rbest = 0.0f, dbest = 0.0f;
  int kbest = 0;
  float l1 = __builtin_inff(), l2 = __builtin_inff(), l3 = __builtin_inff();
  int k1 = -1, k2 = -1;
  bool loose = false;  // some candidate's radius exceeds kObjRel of its score

  __device__ __forceinline__ void add(float o, float r, int k, float d) {
    const bool better = o < best;  // strict: the first of equal minima is kept
    kbest = better ? k : kbest;
    dbest = better ? d : dbest;
    rbest = better ? r : rbest;
    best = better ? o : best;
    const float l = o - r;
    const bool lt1 = l < l1, lt2 = l < l2, lt3 = l < l3;
    l3 = lt2 ? l2 : (lt3 ? l : l3);
    k2 = lt1 ? k1 : (lt2 ? k : k2);
    l2 = lt1 ? l1 : (lt2 ? l : l2);
    k1 = lt1 ? k : k1;
    l1 = lt1 ? l : l1;
    loose |= r > kObjRel * o;
  }
  // The choice is certain when the best interval lies strictly below every other candidate's
  // lower end, and its objective is accurate when its radius is small enough.  False for
  // exact ties, all-zero groups and NaN scores: those groups are re-scored in fp64.
  __device__ __forceinline__ bool clear(bool all_accurate) const {
    const float lo_other = k1 == kbest ? l2 : l1;
    return (best + rbest < lo_other) && (rbest <= kObjRel * best) && !(all_accurate && loose);
  }
};

// Candidates a marked row re-scores: those whose interval reaches below the best interval's
// upper end (the exact minimiser is among them).  Usually that is the best and at most one
// more, which the two smallest lower ends name; when the third smallest also reaches below, or
// every objective is wanted, it is all of them.  The `parts` lanes of a row share the work:
// lane `part` takes the part-th named candidate, or every parts-th index.
struct CandSet {
  int c[2] = {-1, -1};
  bool all = false;
  __device__ __forceinline__ void from(const Track& t) {
    const float upper = t.best + t.rbest;
    all = !(t.l3 > upper);
    c[0] = t.l1 <= upper ? t.k1 : -1;
    c[1] = t.l2 <= upper ? t.k2 : -1;
  }
  // the candidate indices of lane `part`: k = first(), then next(k) until -1
  __device__ __forceinline__ int first(int part, int n_cand) const {
    if (all) return part < n_cand ? part : -1;
    return part < 2 ? c[part] : -1;
  }
  __device__ __forceinline__ int next(int k, int parts, int n_cand) const {
    return (all && k + parts < n_cand) ? k + parts : -1;
  }
};

// Entry p of the upper triangle of a 32x32 block (diagonal included) in row-major order:
// row tri_row(p), column tri_col(p), LDS index 32 row + column.  Compile-time after unrolling.
constexpr int kTri = kGroup * (kGroup + 1) / 2;  // 528
__host__ __device__ constexpr int tri_row(int p) {
  int i = 0;
  while (p >= kGroup - i) {
    p -= kGroup - i;
    ++i;
  }
  return i;
}
__host__ __device__ constexpr int tri_col(int p) {
  int i = 0;
  while (p >= kGroup - i) {
    p -= kGroup - i;
    ++i;
  }
  return i + p;
}
__host__ __device__ constexpr int tri_index(int p) { return kGroup * tri_row(p) + tri_col(p); }
static_assert(tri_row(0) == 0 && tri_col(31) == 31 && tri_row(32) == 1 && tri_col(32) == 1 &&
              tri_row(kTri - 1) == 31 && tri_col(kTri - 1) == 31, "triangle order");

constexpr int kTriChunk = 8, kTriChunks = kTri / kTriChunk;
static_assert(kTri % kTriChunk == 0, "whole chunks");

// one entry of the form: start of row i (diagonal), an off-diagonal term, end of row i
template <int P>
__device__ __forceinline__ void tri_step(double hv, const float (&e)[kGroup], double& s, double& o) {
  constexpr int i = tri_row(P), j = tri_col(P);
  if constexpr (j == i) s = hv * static_cast<double>(e[i]);
  else s = __builtin_fma(hv, static_cast<double>(e[j]), s);
  if constexpr (j == kGroup - 1) o = __builtin_fma(static_cast<double>(e[i]), s, o);
}
template <int P>
constexpr int kTriIndex = tri_index(P);  // a constant expression: never evaluated at run time
template <int C, int... T>
__device__ __forceinline__ void tri_load(const double* hs, int off, double (&b)[kTriChunk],
                                         std::integer_sequence<int, T...>) {
  ((b[T] = hs[off + kTriIndex<C * kTriChunk + T>]), ...);
}
template <int C, int... T>
__device__ __forceinline__ void tri_compute(const double (&b)[kTriChunk], const float (&e)[kGroup],
                                            double& s, double& o, std::integer_sequence<int, T...>) {
  (tri_step<C * kTriChunk + T>(b[T], e, s, o), ...);
}
template <int C>
__device__ __forceinline__ void tri_chunks(const double* hs, int& off, const float (&e)[kGroup],
                                           double (&buf)[2][kTriChunk], double& s, double& o) {
  if constexpr (C + 1 < kTriChunks) {
    asm volatile("" : "+v"(off) : "v"(o), "v"(s));
    tri_load<C + 1>(hs, off, buf[(C + 1) & 1], std::make_integer_sequence<int, kTriChunk>{});
  }
  tri_compute<C>(buf[C & 1], e, s, o, std::make_integer_sequence<int, kTriChunk>{});
  if constexpr (C + 1 < kTriChunks) tri_chunks<C + 1>(hs, off, e, buf, s, o);
}

// fp64 objective of one candidate of one row: e_i = w_i - d * code(w_i, d) (exact in fp32 and
// fp64), obj = sum_i e_i (H_ii e_i + sum_{j > i} (H_ij + H_ji) e_j) in fp64.  hs holds that
// form of the block in LDS: hs[32 i + i] = H_ii, hs[32 i + j] = H_ij + H_ji for j > i (every
// lane reads the same entry at the same time, so the reads are broadcasts).  The errors stay in
// fp32 registers and are widened where they are used, so that the rare re-scoring does not
// raise the register count of the pass-1 loop it shares a kernel with.
__device__ __forceinline__ double score_f64(const float* __restrict__ wrow, float d, const double* hs) {
  // at a zero step e = w whatever the (finite) codes are, so the codes need no special case
  const float inv = __builtin_amdgcn_rcpf(d > 0.0f ? d : 1.0f);
  float e[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; i += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(wrow + i);
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 4; ++t)  // exact: |c| <= 8 and d on the fp16 grid
      e[i + t] = __builtin_fmaf(-code_rcp(vv[t], d, inv), d, vv[t]);
  }
  // The 528 entries of the triangle are taken in row-major order in chunks of 8: the loads of
  // chunk c + 1 are issued before chunk c is computed, at an LDS offset that depends (through an
  // empty asm) on the sums after chunk c - 1, so the compiler can neither hoist them out of the
  // caller's candidate loop nor pull more than two chunks into registers.  The chunks and their
  // entries are expanded at compile time (templates), so every index below is a constant.
  double buf[2][kTriChunk];
  double o = 0.0, s = 0.0;
  int off = 0;
  tri_load<0>(hs, 0, buf[0], std::make_integer_sequence<int, kTriChunk>{});
  tri_chunks<0>(hs, off, e, buf, s, o);
  return o;
}

// Pass 2, at the end of the pass-1 block: fp64 re-scoring of the rows whose pass-1 choice is
// not certain (or whose objective is not accurate enough).  A block covers one group column g,
// so when any of its rows is marked it stages Hg in LDS in fp64 (the symmetric form of
// score_f64).  Each lane then scores, in fp64, the candidates of its row in `cand` that belong
// to its share (the `parts` lanes of a row take every parts-th index), keeping the first
// minimum; the shares are combined across the row's lanes (lane distance `stride`), lowest
// index first on equal objectives, and the first lane of the row writes the results.
// Every thread of the block calls this.
__device__ __forceinline__ void rescore(const float* __restrict__ w, int64_t d_in,
                                        const float* __restrict__ h, int64_t ldh,
                                        const float* __restrict__ alpha, int n_cand,
                                        float* __restrict__ scale, uint8_t* __restrict__ idx,
                                        float* __restrict__ obj, float* __restrict__ obj_all,
                                        int64_t g, int64_t row, float amax, bool marked, bool writer,
                                        const CandSet& cand, int part, int parts, int stride) {
  __shared__ double hs[kGroup * kGroup];
  if (!__syncthreads_or(marked)) return;  // block-uniform
  const int64_t G = d_in / kGroup;
  const float* __restrict__ hg = h + g * kGroup * ldh + g * kGroup;
  for (int t = threadIdx.x; t < kGroup * kGroup; t += kThreads) {
    const int i = t / kGroup, j = t % kGroup;
    double v = 0.0;
    if (j == i) v = static_cast<double>(hg[i * ldh + i]);
    else if (j > i) v = static_cast<double>(hg[i * ldh + j]) + static_cast<double>(hg[j * ldh + i]);
    hs[t] = v;
  }
  __syncthreads();
  const float* __restrict__ wrow = w + row * d_in + g * kGroup;
  const int64_t o_ = row * G + g;
  double best = __builtin_inf();
  int kbest = 0x7FFFFFFF;
  float dbest = 0.0f;
  int k = marked ? cand.first(part, n_cand) : -1;
  while (__builtin_amdgcn_ballot_w64(k >= 0) != 0) {  // wave-uniform exit
    if (k >= 0) {
      const float d = candidate_fast(amax, alpha[k]);  // the step pass 1 used
      const double o = score_f64(wrow, d, hs);
      if (obj_all != nullptr) obj_all[o_ * n_cand + k] = static_cast<float>(o);
      if (o < best || (o == best && k < kbest)) {
        best = o;
        kbest = k;
        dbest = d;
      }
      k = cand.next(k, parts, n_cand);
    }
  }
  for (int off = stride; off < stride * parts; off <<= 1) {
    const double ob = __shfl_xor(best, off);
    const int ok = __shfl_xor(kbest, off);
    const float od = __shfl_xor(dbest, off);
    const bool take = (ob < best) || (ob == best && ok < kbest);
    best = take ? ob : best;
    kbest = take ? ok : kbest;
    dbest = take ? od : dbest;
  }
  if (marked && writer) {
    scale[o_] = dbest;
    idx[o_] = static_cast<uint8_t>(kbest);
    if (obj != nullptr) obj[o_] = static_cast<float>(best);
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
// 16-term fp32 dot per lane plus one exchange with the partner lane.  The same mapping with
// the hi parts of |Hg| and |e| gives B = |e|^T |Hg| |e|, the scale of the score's error.
//
// Precision: w is scaled by a power of two per row (sw) and Hg by one per block (sh), both
// exactly, so that their largest magnitudes sit in [2^14, 2^15); the scaled error
// e = sw w - code * (sw D) is exact in fp32 and |e| <= |sw w| (a code never overshoots w by
// more than D / 2 <= |w|, and a clamped or zero code only shrinks w), so nothing overflows fp16.
// e and Hg are each split into two fp16 parts (relative residual <= 2^-22 in fp16's normal
// range), and D accumulates hi*lo, lo*hi, then hi*hi in fp32 (products of fp16 values are
// exact; the dropped lo*lo term is <= 2^-22 relative).  Scores are compared in the scaled
// units (the same factor 2^-(2 log2 sw + log2 sh) for every candidate of a row) and unscaled
// exactly for the outputs.  The headroom matters when the channel scales of X spread widely:
// the block's small entries then lie many binades below its largest one.
//
// Marking: a row is re-scored in fp64 (pass 2) unless its choice is certain and its objective
// accurate by the radii (Track::clear).  Pass 2 scores the candidates of CandSet.  With
// obj_all, every candidate's objective must be accurate, and a marked row's candidates are all
// re-scored.
template <bool kAll>
__global__ __launch_bounds__(kThreads, 4) void search_split_kernel(
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

  // exact power-of-two scalings, then the two fp16 parts of the block (A operands) and the
  // magnitudes of the hi parts (A operands of the bound)
  const int ew = scale_exp(amax), eh = scale_exp(hmax);
  const float sw = pow2(ew), sh = pow2(eh);
  const int unscale = -(2 * ew + eh);  // obj = score * 2^unscale
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    wv[i] *= sw;
    ha[i] *= sh;
  }
  f16x8 hhi[2], hlo[2], habs[2];
  split8(ha, hhi[0], hlo[0]);
  split8(ha + 8, hhi[1], hlo[1]);
#pragma unroll
  for (int u = 0; u < 2; ++u) habs[u] = abs8(hhi[u]);

  // score and radius of candidate step d (scaled units; same bits in both lanes of a row)
  auto eval = [&](float d, float& o, float& rad) {
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
    const f16x8 eabs[2] = {abs8(ehi[0]), abs8(ehi[1])};
    float p0 = 0.0f, p1 = 0.0f;  // even and odd positions of the lane
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      p0 = __builtin_fmaf(e[i], acc[i], p0);
      p1 = __builtin_fmaf(e[i + 1], acc[i + 1], p1);
    }
    // the bound's products reuse the registers of the score's accumulator
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(habs[u], eabs[u], acc, 0, 0, 0);
    float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      b0 = __builtin_fmaf(__builtin_fabsf(e[i]), acc[i], b0);
      b1 = __builtin_fmaf(__builtin_fabsf(e[i + 1]), acc[i + 1], b1);
    }
    o = pair_sum32(p0 + p1);
    rad = kRad * pair_sum32(b0 + b1);
  };

  Track t;
  float d_next = candidate_fast(amax, alpha[0]);
#pragma unroll 1
  for (int k = 0; k < n_cand; ++k) {
    const float d = d_next;
    // the next candidate's step, off this candidate's dependency chain
    d_next = candidate_fast(amax, alpha[k + 1 < n_cand ? k + 1 : k]);
    float o, rad;
    eval(d, o, rad);
    if (kAll && live && hh == 0) obj_all[(r * G + g) * n_cand + k] = __builtin_ldexpf(o, unscale);
    t.add(o, rad, k, d);
  }
  const bool clear = t.clear(kAll);
  const bool writer = live && hh == 0;
  if (writer && clear) {
    const int64_t o_ = r * G + g;
    scale[o_] = t.dbest;
    idx[o_] = static_cast<uint8_t>(t.kbest);
    if (obj != nullptr) obj[o_] = __builtin_ldexpf(t.best, unscale);
  }
  const bool marked = live && !clear;
  CandSet cand;
  cand.from(t);
  cand.all |= kAll;
  rescore(w, d_in, h, ldh, alpha, n_cand, scale, idx, obj, obj_all, g, rr, amax, marked, writer,
          cand, hh, 2, 32);
}

// Pass 1 for small grids: 16 rows per wavefront (twice the wavefronts of the kernel above, so
// short problems still fill the SIMDs).  Lane (q, j) = (lane / 16, lane % 16) owns positions
// p = 8 q + e (e = 0..7) of row j.  v_mfma_f32_32x32x16_f16 is replaced by pairs of
// v_mfma_f32_16x16x32_f16: product u (0, 1) has output rows i = 0..15 standing for positions
// 8 (i / 4) + 4 u + i % 4 and the reduction slot 8 q + e standing for position 8 q + e, so the
// lane feeds its own 8 errors as the B operand and Hg[8 (i / 4) + 4 u + i % 4][8 q + e] (i = the
// lane's j) as the A operand, and receives D[p][j] for exactly its own positions
// p = 8 q + 4 u + r (r = 0..3).  Scaling, splitting, accumulation order, radii and marking as
// above; the four lanes of a row share pass 2's candidates.
template <bool kAll>
__global__ __launch_bounds__(kThreads, 4) void search_split16_kernel(
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
  f16x8 hhi[2], hlo[2], habs[2];
  split8(ha[0], hhi[0], hlo[0]);
  split8(ha[1], hhi[1], hlo[1]);
#pragma unroll
  for (int u = 0; u < 2; ++u) habs[u] = abs8(hhi[u]);

  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  auto eval = [&](float d, float& o, float& rad) {
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
    const f16x8 eabs = abs8(ehi);
    f32x4 acc[2], accb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hhi[u], elo, zero4, 0, 0, 0);
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hlo[u], ehi, acc[u], 0, 0, 0);
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hhi[u], ehi, acc[u], 0, 0, 0);
      accb[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(habs[u], eabs, zero4, 0, 0, 0);
    }
    float p0 = 0.0f, p1 = 0.0f, b0 = 0.0f, b1 = 0.0f;  // two chains: the two products
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0 = __builtin_fmaf(e[i], acc[0][i], p0);
      p1 = __builtin_fmaf(e[4 + i], acc[1][i], p1);
      b0 = __builtin_fmaf(__builtin_fabsf(e[i]), accb[0][i], b0);
      b1 = __builtin_fmaf(__builtin_fabsf(e[4 + i]), accb[1][i], b1);
    }
    o = quad_sum(p0 + p1);
    rad = kRad * quad_sum(b0 + b1);
  };

  Track t;
  float d_next = candidate_fast(amax, alpha[0]);
#pragma unroll 1
  for (int k = 0; k < n_cand; ++k) {
    const float d = d_next;
    // the next candidate's step, off this candidate's dependency chain
    d_next = candidate_fast(amax, alpha[k + 1 < n_cand ? k + 1 : k]);
    float o, rad;
    eval(d, o, rad);
    if (kAll && live && q == 0) obj_all[(r * G + g) * n_cand + k] = __builtin_ldexpf(o, unscale);
    t.add(o, rad, k, d);
  }
  const bool clear = t.clear(kAll);
  const bool writer = live && q == 0;
  if (writer && clear) {
    const int64_t o_ = r * G + g;
    scale[o_] = t.dbest;
    idx[o_] = static_cast<uint8_t>(t.kbest);
    if (obj != nullptr) obj[o_] = __builtin_ldexpf(t.best, unscale);
  }
  const bool marked = live && !clear;
  CandSet cand;
  cand.from(t);
  cand.all |= kAll;
  rescore(w, d_in, h, ldh, alpha, n_cand, scale, idx, obj, obj_all, g, rr, amax, marked, writer,
          cand, q, 4, 16);
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

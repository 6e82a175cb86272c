// gptq.hip -- GPTQ error feedback on the group-32 grid with fixed steps (static groups).
//
// GPTQ (Frantar et al., "GPTQ: Accurate Post-Training Quantization for Generative Pre-trained
// Transformers", the published algorithm) is the second-order output reconstruction method the
// blog "Opt.Gear-QAT: Preserving On-Device Performance with QAT", section 2, starts from.  With
// H' = H (dead columns: unit diagonal, zero weight) + damp * mean(diag) I, the columns of a row are
// quantized in order, each from the least-squares update of the not-yet-quantized weights given
// the ones already quantized.  The published form feeds err_i = (w'_i - w_hat_i) / U_ii through
// U = chol(H'^-1)^T.  Here the same updated weights come from the Cholesky factor of H' itself,
// without the inverse: with H' = R R^T, R upper (R = J L J for J H' J = L L^T, J the reversal),
//   w'_i = w_i + (1 / R_ii) sum_{p < i} R_pi (w_p - w_hat_p),
// (U = R^-1 gives U^T U = H'^-1, and (w - w_hat) = U^T err unrolls to the sum above).  So:
//   1. A = J H' J in fp64, dp x dp (dp = d_in rounded up to 64, identity beyond d_in);
//   2. blocked Cholesky A = L L^T (panels of 64: a one-workgroup diagonal factor, a wavefront per
//      row for the panel below it, and the trailing update on the fp64 matrix cores);
//   3. per block of 64 columns: the sums over earlier columns on the matrix cores
//      (delta [rows][c0] times R [c0][block]), then the block's columns in order inside the
//      workgroup, delta_i = w_i - w_hat_i kept in fp64 for the later blocks.
// Everything runs in fp64; codes follow the exact nearest-code rule on the fp64 updated weight.
#include "common.hpp"

namespace w4q {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

constexpr int kNb = 64;  // panel and column-block width

// nearest code of the fp64 value v at step d (fp32, >= 0; inv_d ~ 1 / d): ties to the even code,
// clamped.  The first guess rint(v inv_d) is within one code of the answer; (c +- 1/2) d is exact in
// fp64 and v - (c +- 1/2) d has the sign of the exact difference, which settles it.
__device__ __forceinline__ double code64(double v, double d, double inv_d) {
  if (!(d > 0.0)) return 0.0;
  double c = __builtin_rint(v * inv_d);
  c = __builtin_fmin(__builtin_fmax(c, -8.0), 7.0);
  const double rh = v - (c + 0.5) * d;
  const double rl = v - (c - 0.5) * d;
  const bool odd = (static_cast<int>(c) & 1) != 0;
  const bool up = (rh > 0.0 || (rh == 0.0 && odd)) && c < 7.0;
  const bool dn = (rl < 0.0 || (rl == 0.0 && odd)) && c > -8.0;
  return c + (up ? 1.0 : 0.0) - (dn ? 1.0 : 0.0);
}

// ------------------------------------------------------------------------------ prep
// mean of the diagonal with dead entries read as 1 (one workgroup, fixed summation order)
__global__ __launch_bounds__(256) void diag_mean_kernel(const float* __restrict__ h, int64_t ldh, int64_t d,
                                                        double* __restrict__ mean) {
  __shared__ double part[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 256) {
    const double v = static_cast<double>(h[i * ldh + i]);
    s += v == 0.0 ? 1.0 : v;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k >= 1; k >>= 1) {
    if (static_cast<int>(threadIdx.x) < k) part[threadIdx.x] += part[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) *mean = part[0] / static_cast<double>(d);
}

// A[i][j] = H'[d-1-i][d-1-j] inside d x d, identity beyond; dead[k] = (H_kk == 0)
__global__ __launch_bounds__(256) void build_kernel(const float* __restrict__ h, int64_t ldh, int64_t d, int64_t dp,
                                                    const double* __restrict__ mean, float damp,
                                                    double* __restrict__ a, uint8_t* __restrict__ dead) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= dp * dp) return;
  const int64_t i = e / dp, j = e % dp;
  double v;
  if (i < d && j < d) {
    const int64_t hi = d - 1 - i, hj = d - 1 - j;
    v = static_cast<double>(h[hi * ldh + hj]);
    if (i == j) {
      if (v == 0.0) v = 1.0;
      v += static_cast<double>(damp) * *mean;
    }
  } else {
    v = i == j ? 1.0 : 0.0;
  }
  a[e] = v;
  if (i == j && i < d) dead[d - 1 - i] = h[(d - 1 - i) * ldh + (d - 1 - i)] == 0.0f ? 1 : 0;
}

// --------------------------------------------------------------------- blocked Cholesky
// diagonal block [k0, k0 + 64), right-looking: thread (i, m) = (tid / 4, tid % 4) keeps entries
// (i, 16 m .. 16 m + 15) of the block in registers; for column j its owners (m = j / 16) publish
// column j through LDS (two buffers, so one barrier per column), every thread then updates its
// entries by L_ij L_kj and the owners record L_ij.  A pivot that is not positive sets *info.
__global__ __launch_bounds__(256) void chol_diag_kernel(double* __restrict__ a, int64_t dp, int64_t k0,
                                                        int* __restrict__ info) {
  __shared__ double colbuf[2][kNb];
  __shared__ double lo[kNb][kNb + 1];
  const int tid = threadIdx.x, i = tid >> 2, m = tid & 3;
  double t[16];
  const double* arow = a + (k0 + i) * dp + k0 + 16 * m;
#pragma unroll
  for (int c = 0; c < 16; c += 2) {
    const f64x2 v = *reinterpret_cast<const f64x2*>(arow + c);
    t[c] = v.x;
    t[c + 1] = v.y;
  }
  for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int j = 16 * jb + c, b = c & 1;
      if (m == jb) colbuf[b][i] = t[c];
      __syncthreads();
      const double p = colbuf[b][j];
      const double aij = colbuf[b][i];
      if (tid == 0 && !(p > 0.0) && info != nullptr) *info = 1;
      // L_ij L_kj = a_ij a_kj / p: one division on the path from column to column.  All 16 entries
      // are updated: only those in (j, i] are read again (published columns are j + 1 .. 63, and
      // rows i <= j only ever feed their own unused entries), so no masks are needed.
      const double f = aij / p;
#pragma unroll
      for (int c2 = 0; c2 < 16; ++c2) t[c2] = __builtin_fma(-f, colbuf[b][16 * m + c2], t[c2]);
      if (m == jb && i >= j) {  // the factor's entry, off that path
        const double dj = __builtin_sqrt(p);
        lo[i][j] = i == j ? dj : aij / dj;
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < kNb * kNb; e += 256) {
    const int r = e / kNb, k = e % kNb;
    if (k <= r) a[(k0 + r) * dp + k0 + k] = lo[r][k];
  }
}

// panel below the diagonal block: row i solves x L11^T = a_i (one wavefront per row, lane j
// holds x_j; the columns are settled in order, x_j = s_j / L_jj (by the lane's reciprocal of its
// pivot) taken from lane j by readlane)
__global__ __launch_bounds__(256) void chol_panel_kernel(double* __restrict__ a, int64_t dp, int64_t k0) {
  __shared__ double l[kNb][kNb + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int e = tid; e < kNb * kNb; e += 256) l[e / kNb][e % kNb] = a[(k0 + e / kNb) * dp + k0 + e % kNb];
  __syncthreads();
  const int64_t row = k0 + kNb + static_cast<int64_t>(blockIdx.x) * 4 + (tid >> 6);
  if (row >= dp) return;  // uniform per wavefront; no barrier follows
  double s = a[row * dp + k0 + lane];
  const double rdiag = 1.0 / l[lane][lane];
  double x = 0.0;
  for (int j = 0; j < kNb; ++j) {
    const double q = s * rdiag;  // lane j's value is x_j
    const uint64_t qb = __builtin_bit_cast(uint64_t, q);
    const uint32_t lo32 = __builtin_amdgcn_readlane(static_cast<uint32_t>(qb), j);
    const uint32_t hi32 = __builtin_amdgcn_readlane(static_cast<uint32_t>(qb >> 32), j);
    const double xj = __builtin_bit_cast(double, (static_cast<uint64_t>(hi32) << 32) | lo32);
    if (lane == j) x = xj;
    if (lane > j) s -= xj * l[lane][j];
  }
  a[row * dp + k0 + lane] = x;
}

// trailing update of the lower tile pairs: A[ti][tj] -= L21[ti] L21[tj]^T (K = 64), tiles of 64
// rows past k0 + 64, ti >= tj; 16 rows x 64 columns per wavefront.  Every operand and the 16
// target entries of a lane are loaded before the first product (one round trip per launch).
__global__ __launch_bounds__(256) void chol_update_kernel(double* __restrict__ a, int64_t dp, int64_t k0) {
  // tile pair of this workgroup: b = ti (ti + 1) / 2 + tj
  const int64_t b = blockIdx.x;
  int64_t ti = static_cast<int64_t>((__builtin_sqrt(8.0 * static_cast<double>(b) + 1.0) - 1.0) * 0.5);
  while ((ti + 1) * (ti + 2) / 2 <= b) ++ti;
  while (ti * (ti + 1) / 2 > b) --ti;
  const int64_t tj = b - ti * (ti + 1) / 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int64_t base = k0 + kNb;
  const int64_t ra = base + ti * kNb + 16 * wave + j;  // A-side row
  const double* arow = a + ra * dp + k0;
  double av[16], bv[4][16], tv[4][4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const f64x2 a01 = *reinterpret_cast<const f64x2*>(arow + 16 * st + 4 * q);
    const f64x2 a23 = *reinterpret_cast<const f64x2*>(arow + 16 * st + 4 * q + 2);
    av[4 * st] = a01.x;
    av[4 * st + 1] = a01.y;
    av[4 * st + 2] = a23.x;
    av[4 * st + 3] = a23.y;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const double* brow = a + (base + tj * kNb + 16 * c + j) * dp + k0 + 16 * st + 4 * q;
      const f64x2 b01 = *reinterpret_cast<const f64x2*>(brow);
      const f64x2 b23 = *reinterpret_cast<const f64x2*>(brow + 2);
      bv[c][4 * st] = b01.x;
      bv[c][4 * st + 1] = b01.y;
      bv[c][4 * st + 2] = b23.x;
      bv[c][4 * st + 3] = b23.y;
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = base + ti * kNb + 16 * wave + 4 * r + q;
      const int64_t col = base + tj * kNb + 16 * c + j;
      tv[c][r] = a[row * dp + col];
    }
  asm volatile("" ::: "memory");
  f64x4 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < 16; ++s)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[s], bv[c][s], acc[c], 0, 0, 0);
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = base + ti * kNb + 16 * wave + 4 * r + q;
      const int64_t col = base + tj * kNb + 16 * c + j;
      a[row * dp + col] = tv[c][r] - acc[c][r];
    }
}

// ------------------------------------------------------------------------------ sweep
// R[p][i] = L[d-1-p][d-1-i] (p <= i): the upper factor of H' read through the reversal
__device__ __forceinline__ double rfac(const double* __restrict__ l, int64_t dp, int64_t d, int64_t p, int64_t i) {
  return l[(d - 1 - p) * dp + (d - 1 - i)];
}

// Block of columns [c0, c0 + nb) for 16 rows per workgroup (16 wavefronts).  First the sums over
// the earlier columns on the matrix cores: wavefront w takes block columns 16 (w % 4) .. + 15 and
// every fourth 16-column step of the earlier columns from step w / 4 on (loads of the next step
// issued before the products of the current one); the four partial sums of an entry are added in
// LDS in a fixed order.  Then each wavefront takes one of the 16 rows, a lane per block column,
// and the block's columns are quantized in order with the correction of every later column of
// the block kept current.
constexpr int kBlockThreads = 1024;

__global__ __launch_bounds__(kBlockThreads) void gptq_block_kernel(const float* __restrict__ w, int64_t d_out,
                                                                   int64_t d_in, const float* __restrict__ scale,
                                                                   const double* __restrict__ l, int64_t dp,
                                                                   const uint8_t* __restrict__ dead,
                                                                   double* __restrict__ delta,
                                                                   float* __restrict__ w_hat, int64_t c0) {
  __shared__ double part[4][16][kNb + 1];
  __shared__ double rd[kNb][kNb + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int cg = wave & 3, kq = wave >> 2;
  const int64_t G = d_in / kGroup;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int nb = d_in - c0 < kNb ? static_cast<int>(d_in - c0) : kNb;
  // 1. partial C[row][c0 + 16 cg + j] over the steps kk0 = 16 (kq + 4 n) < c0.  Rows past d_out and
  //    columns past d_in read the last valid ones (their sums are never used), so every load is
  //    unconditional and the next step's loads stay in flight across the current products.
  {
    const int64_t ra = r0 + j < d_out ? r0 + j : d_out - 1;
    const double* drow = delta + ra * d_in + 4 * q;
    const int64_t col = c0 + 16 * cg + j < d_in ? c0 + 16 * cg + j : d_in - 1;
    // R[p][col] = L[d-1-p][d-1-col]: rows p = kk0 + 4 q + s
    const double* rcol = l + (d_in - 1 - 4 * q) * dp + (d_in - 1 - col);
    f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
    double av[4], bv[4], an[4], bn[4];
    auto fetch = [&](int64_t kk0, double* ao, double* bo) {
      const f64x2 a01 = *reinterpret_cast<const f64x2*>(drow + kk0);
      const f64x2 a23 = *reinterpret_cast<const f64x2*>(drow + kk0 + 2);
      ao[0] = a01.x;
      ao[1] = a01.y;
      ao[2] = a23.x;
      ao[3] = a23.y;
#pragma unroll
      for (int s = 0; s < 4; ++s) bo[s] = rcol[-(kk0 + s) * dp];
    };
    // this wavefront's steps kk0 = 16 kq + 64 n, n < ns; the fetch of step n + 1 (clamped to the
    // last step) is issued before the products of step n, the compiler fences keep it there.
    // (Three steps in flight measured no faster: 4096 x 4096 8.47 vs 8.38 ms.)
    const int64_t ns = 16 * kq < c0 ? (c0 - 16 * kq + 63) / 64 : 0;
    auto kstep = [&](int64_t n) { return 16 * kq + 64 * (n < ns - 1 ? n : ns - 1); };
    auto mma = [&](const double* ao, const double* bo) {
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(ao[s], bo[s], acc, 0, 0, 0);
    };
    if (ns > 0) {  // uniform per wavefront
      fetch(kstep(0), av, bv);
      for (int64_t n = 0; n < ns; n += 2) {
        fetch(kstep(n + 1), an, bn);
        asm volatile("" ::: "memory");
        mma(av, bv);
        if (n + 1 >= ns) break;
        fetch(kstep(n + 2), av, bv);
        asm volatile("" ::: "memory");
        mma(an, bn);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) part[kq][4 * r + q][16 * cg + j] = acc[r];
  }
  // 2. the block's diagonal part of R
  for (int e = tid; e < kNb * kNb; e += kBlockThreads) {
    const int i = e / kNb, k = e % kNb;
    rd[i][k] = (i <= k && i < nb && k < nb) ? rfac(l, dp, d_in, c0 + i, c0 + k) : 0.0;
  }
  __syncthreads();
  // 3. the block's columns in order: wavefront w takes row r0 + w, lane k block column k.  Column
  //    i is quantized by lane i; its delta reaches every lane by readlane and corrects the later
  //    columns.  Each lane keeps its own column's results and stores them at the end.
  const int64_t row = r0 + wave;
  if (row >= d_out) return;  // uniform per wavefront; no barrier follows
  const int k = lane;
  const bool in = k < nb;
  double cl = ((part[0][wave][k] + part[1][wave][k]) + part[2][wave][k]) + part[3][wave][k];
  const double wl = (in && dead[c0 + k] == 0) ? static_cast<double>(w[row * d_in + c0 + k]) : 0.0;
  const double d = in ? static_cast<double>(scale[row * G + (c0 + k) / kGroup]) : 0.0;
  const double inv_d = d > 0.0 ? 1.0 / d : 0.0;
  const double inv_r = in ? 1.0 / rd[k][k] : 0.0;
  double wh_k = 0.0, di_k = 0.0;
  for (int i = 0; i < nb; ++i) {
    // every lane evaluates its own column; lane i's is the one taken
    const double v = wl + cl * inv_r;
    const double wh = d * code64(v, d, inv_d);
    const double di = wl - wh;
    if (k == i) {
      wh_k = wh;
      di_k = di;
    }
    const uint64_t bits = __builtin_bit_cast(uint64_t, di);
    const uint32_t lo32 = __builtin_amdgcn_readlane(static_cast<uint32_t>(bits), i);
    const uint32_t hi32 = __builtin_amdgcn_readlane(static_cast<uint32_t>(bits >> 32), i);
    const double dii = __builtin_bit_cast(double, (static_cast<uint64_t>(hi32) << 32) | lo32);
    if (k > i) cl = __builtin_fma(rd[i][k], dii, cl);
  }
  if (in) {
    w_hat[row * d_in + c0 + k] = static_cast<float>(wh_k);
    delta[row * d_in + c0 + k] = di_k;
  }
}

inline unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }
inline size_t up256(size_t b) { return (b + 255) & ~size_t(255); }

}  // namespace
}  // namespace w4q

using namespace w4q;

size_t w4q_gptq_workspace(int64_t d_out, int64_t d_in) {
  const int64_t dp = (d_in + 63) & ~int64_t(63);
  return up256(static_cast<size_t>(dp * dp) * 8) + up256(static_cast<size_t>(d_out * d_in) * 8) +
         up256(static_cast<size_t>(d_in)) + 256;
}

int w4q_launch_gptq(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh, const float* scale,
                    float damp, float* w_hat, int* info, void* ws, hipStream_t s) {
  const int64_t dp = (d_in + 63) & ~int64_t(63);
  char* p = static_cast<char*>(ws);
  double* a = reinterpret_cast<double*>(p);
  p += up256(static_cast<size_t>(dp * dp) * 8);
  double* delta = reinterpret_cast<double*>(p);
  p += up256(static_cast<size_t>(d_out * d_in) * 8);
  uint8_t* dead = reinterpret_cast<uint8_t*>(p);
  p += up256(static_cast<size_t>(d_in));
  double* mean = reinterpret_cast<double*>(p);
  int rc;
#define W4Q_GO(...)                                  \
  do {                                               \
    hipLaunchKernelGGL(__VA_ARGS__);                 \
    if ((rc = w4q_launch_status()) != W4Q_OK) return rc; \
  } while (0)
  W4Q_GO(diag_mean_kernel, dim3(1), dim3(256), 0, s, h, ldh, d_in, mean);
  W4Q_GO(build_kernel, dim3(cdiv(dp * dp, 256)), dim3(256), 0, s, h, ldh, d_in, dp, mean, damp, a, dead);
  for (int64_t k0 = 0; k0 < dp; k0 += kNb) {
    W4Q_GO(chol_diag_kernel, dim3(1), dim3(256), 0, s, a, dp, k0, info);
    const int64_t rest = dp - k0 - kNb;
    if (rest > 0) {
      W4Q_GO(chol_panel_kernel, dim3(cdiv(rest, 4)), dim3(256), 0, s, a, dp, k0);
      const int64_t T = rest / kNb;
      W4Q_GO(chol_update_kernel, dim3(static_cast<unsigned>(T * (T + 1) / 2)), dim3(256), 0, s, a, dp, k0);
    }
  }
  for (int64_t c0 = 0; c0 < d_in; c0 += kNb)
    W4Q_GO(gptq_block_kernel, dim3(cdiv(d_out, 16)), dim3(kBlockThreads), 0, s, w, d_out, d_in, scale, a, dp, dead,
           delta, w_hat, c0);
#undef W4Q_GO
  return W4Q_OK;
}

// joint.hip -- quadratic forms with the full H in fp64: the per-channel scale search, the joint
// (whole-row) objective of a group-32 choice, and coordinate descent over the groups of a row.
//
// Method: model card "Opt.Gear-1B-qat-int4-per-channel-unquantized", "Quantization
// Configuration": the step minimises ||W X - Q(W) X||_F^2, which for output row w is e^T H e with
// e = w - Q(w) and H = X^T X.  The group search (scale_search.hip) reads it per group of 32 with
// the diagonal blocks of H, so the groups are independent.  Read over a whole row, the
// off-diagonal blocks couple them:
//   * per-channel (the card's own checkpoint: one scale per output row): every candidate's
//     e^T H e with the full H, first minimum;
//   * joint objective of a group-32 choice: e^T H e over the row;
//   * coordinate descent: the groups of a row in order, each group's candidates tried with the
//     others held; trial k of group g changes the objective by
//     dO = 2 d^T u_g + d^T H_gg d,  d = e_g(k) - e_g,  u = H e,
//     and after a change u += H[:, g] d.
//
// Arithmetic: e = w - D q is exact in fp64 (D an fp32 step, q an integer code by the exact
// nearest-code rule), H entries are the fp32 values given, and every product and sum runs in
// fp64, on the matrix cores (v_mfma_f64_16x16x4f64) for the dense products E H and in fp64 FMAs
// for the per-group trials.
//
// Matrix-core layout (16x16x4 fp64): lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16];
// result register r of lane l holds D[4r + l / 16][l % 16].  The reduction index of a 16-deep
// tile is assigned as kk = 4 (l / 16) + s for step s, so that a lane's four A values are four
// consecutive weights (one 16-byte load); the B operand follows the same assignment.
#include "common.hpp"

namespace w4q {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 16;   // reduction rows of H per staged tile
constexpr int kBN = 64;   // columns per block: four 16-wide matrix-core tiles
constexpr int kLdt = 68;  // LDS row stride (floats): the four lane quarters read distinct banks

// e = w - d * code(w, d), exact in fp64 (d = 0: code 0)
__device__ __forceinline__ double err(float w, float d, float inv) {
  const float q = d > 0.0f ? code_rcp(w, d, inv) : 0.0f;
  return static_cast<double>(w) - static_cast<double>(d) * static_cast<double>(q);
}

__device__ __forceinline__ float inv_of(float d) { return d > 0.0f ? 1.0f / d : 0.0f; }

// Stages rows kk0..kk0+BK-1, columns c0..c0+63 of H (zeros past column d) through registers:
// fetch() issues the loads of this thread's share, put() writes them to an LDS buffer.
template <int NT, int BK = kBK>
struct Stager {
  static constexpr int kTileF4 = BK * kBN / 4;  // float4 loads per tile
  static constexpr int kPer = (kTileF4 + NT - 1) / NT;
  f32x4 r[kPer];
  __device__ __forceinline__ void fetch(const float* __restrict__ h, int64_t ldh, int64_t d, int64_t kk0,
                                        int64_t c0, int tid) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int i = tid + p * NT;
      const int row = i / (kBN / 4), f = i % (kBN / 4);
      const int64_t col = c0 + 4 * f;
      r[p] = (i < kTileF4 && col < d) ? *reinterpret_cast<const f32x4*>(h + (kk0 + row) * ldh + col)
                                       : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
  __device__ __forceinline__ void put(float* t, int tid) const {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int i = tid + p * NT;
      if (i < kTileF4) {
        const int row = i / (kBN / 4), f = i % (kBN / 4);
        *reinterpret_cast<f32x4*>(t + row * kLdt + 4 * f) = r[p];
      }
    }
  }
};

// acc[c] += A B_c over one staged tile: a[s] is this lane's A value for step s
__device__ __forceinline__ void tile_mma(const float* t, const double (&a)[4], f64x4 (&acc)[4], int lane) {
  const int q = lane >> 4, j = lane & 15;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const double b = static_cast<double>(t[(4 * q + s) * kLdt + 16 * c + j]);
      acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s], b, acc[c], 0, 0, 0);
    }
}

// sum over the 16 lanes l % 16 = 0..15 of a quarter (fixed order); every lane gets the sum
__device__ __forceinline__ double quarter_sum(double v) {
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 1);
  return v;
}

// ------------------------------------------------------------------ per-channel search
// One workgroup per output row; its candidates are the rows of E, 16 per wavefront, in blocks
// of 16 NW.  For each block of 64 columns the product T = E H[:, cols] is accumulated over the
// whole reduction, then e . T over those columns is added to each candidate's objective.
template <int NW>
__global__ __launch_bounds__(64 * NW) void pc_search_kernel(const float* __restrict__ w, int64_t d_in,
                                                             const float* __restrict__ h, int64_t ldh,
                                                             const float* __restrict__ alpha, int n_cand,
                                                             float* __restrict__ scale, uint8_t* __restrict__ idx,
                                                             float* __restrict__ obj, float* __restrict__ obj_all) {
  constexpr int NT = 64 * NW;
  constexpr int kPcBK = 2 * kBK;  // H rows per staged tile: two matrix-core steps per barrier
  __shared__ float tile[2][kPcBK * kLdt];
  __shared__ double objs[256];
  __shared__ float wmax[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int64_t row = blockIdx.x;
  const float* wrow = w + row * d_in;

  float m = 0.0f;
  for (int64_t i = tid; i < d_in; i += NT) m = __builtin_fmaxf(m, __builtin_fabsf(wrow[i]));
  for (int off = 32; off >= 1; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  float amax = wmax[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) amax = __builtin_fmaxf(amax, wmax[i]);

  const int nkb = static_cast<int>(d_in / kPcBK);  // d_in % 32 == 0
  Stager<NT, kPcBK> st;
  for (int cb = 0; cb < n_cand; cb += 16 * NW) {
    const int ka = cb + 16 * wave + j;  // this lane's A-side candidate
    const float da = ka < n_cand ? candidate(amax, alpha[ka]) : 0.0f;
    const float ia = inv_of(da);
    float de[4], ie[4];  // result-side candidates cb + 16 wave + 4r + q
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = cb + 16 * wave + 4 * r + q;
      de[r] = k < n_cand ? candidate(amax, alpha[k]) : 0.0f;
      ie[r] = inv_of(de[r]);
    }
    double part[4] = {0.0, 0.0, 0.0, 0.0};
    for (int64_t c0 = 0; c0 < d_in; c0 += kBN) {
      f64x4 acc[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = f64x4{0.0, 0.0, 0.0, 0.0};
      st.fetch(h, ldh, d_in, 0, c0, tid);
      st.put(tile[0], tid);
      __syncthreads();
      for (int t = 0; t < nkb; ++t) {
        const int64_t kk0 = static_cast<int64_t>(t) * kPcBK;
        if (t + 1 < nkb) st.fetch(h, ldh, d_in, kk0 + kPcBK, c0, tid);
#pragma unroll
        for (int sub = 0; sub < kPcBK / kBK; ++sub) {
          const f32x4 wv = *reinterpret_cast<const f32x4*>(wrow + kk0 + kBK * sub + 4 * q);
          const double a[4] = {err(wv.x, da, ia), err(wv.y, da, ia), err(wv.z, da, ia), err(wv.w, da, ia)};
          tile_mma(tile[t & 1] + kBK * sub * kLdt, a, acc, lane);
        }
        if (t + 1 < nkb) st.put(tile[(t + 1) & 1], tid);
        __syncthreads();
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int64_t col = c0 + 16 * c + j;
        if (col < d_in) {
          const float wc = wrow[col];
#pragma unroll
          for (int r = 0; r < 4; ++r) part[r] += acc[c][r] * err(wc, de[r], ie[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const double v = quarter_sum(part[r]);
      const int k = cb + 16 * wave + 4 * r + q;
      if (j == 0 && k < n_cand) objs[k] = v;
    }
  }
  __syncthreads();
  if (obj_all != nullptr)
    for (int k = tid; k < n_cand; k += NT) obj_all[row * n_cand + k] = static_cast<float>(objs[k]);
  if (tid == 0) {
    int kb = 0;
    for (int k = 1; k < n_cand; ++k)
      if (objs[k] < objs[kb]) kb = k;  // strict: the first minimum wins
    scale[row] = candidate(amax, alpha[kb]);
    idx[row] = static_cast<uint8_t>(kb);
    if (obj != nullptr) obj[row] = static_cast<float>(objs[kb]);
  }
}

// ------------------------------------------------------------------------ joint form
// steps[r][g] = candidate(amax of group g of row r, alpha[idx[r][g]]); indices past the
// candidate list are read as its last entry
__global__ __launch_bounds__(256) void steps_kernel(const float* __restrict__ w, int64_t d_in, int64_t rows,
                                                    const float* __restrict__ alpha, int n_cand,
                                                    const uint8_t* __restrict__ idx, float* __restrict__ steps) {
  const int64_t G = d_in / kGroup;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * G) return;
  const float* wg = w + (i / G) * d_in + (i % G) * kGroup;
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < kGroup; k += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(wg + k);
    m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)),
                                           __builtin_fmaxf(__builtin_fabsf(v.z), __builtin_fabsf(v.w))));
  }
  const int k = idx[i] < n_cand ? idx[i] : n_cand - 1;
  steps[i] = candidate(m, alpha[k]);
}

// U = E H for 64 rows per workgroup (16 per wavefront) over the column blocks
// [blockIdx.y * cbs, (blockIdx.y + 1) * cbs); E from the rows' fp32 steps.  Stores U (kStoreU)
// and each row's partial e . U over those columns: part[row][blockIdx.y].
template <bool kStoreU>
__global__ __launch_bounds__(256) void joint_u_kernel(const float* __restrict__ w, const float* __restrict__ steps,
                                                      int64_t rows, int64_t d_in, const float* __restrict__ h,
                                                      int64_t ldh, int cbs, double* __restrict__ u,
                                                      double* __restrict__ part, int n_split) {
  constexpr int NT = 256;
  __shared__ float tile[2][kBK * kLdt];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int64_t G = d_in / kGroup;
  const int64_t rb = static_cast<int64_t>(blockIdx.x) * 64 + 16 * wave;
  const int64_t ra = rb + j;  // this lane's A-side row
  const bool va = ra < rows;
  const float* wa = w + (va ? ra : 0) * d_in;
  const float* sa = steps + (va ? ra : 0) * G;
  const int nkb = static_cast<int>(d_in / kBK);
  const int64_t ncb = (d_in + kBN - 1) / kBN;
  const int64_t cbeg = static_cast<int64_t>(blockIdx.y) * cbs;
  const int64_t cend = cbeg + cbs < ncb ? cbeg + cbs : ncb;
  double p[4] = {0.0, 0.0, 0.0, 0.0};
  Stager<NT> st;
  for (int64_t cbk = cbeg; cbk < cend; ++cbk) {
    const int64_t c0 = cbk * kBN;
    f64x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f64x4{0.0, 0.0, 0.0, 0.0};
    st.fetch(h, ldh, d_in, 0, c0, tid);
    st.put(tile[0], tid);
    __syncthreads();
    for (int t = 0; t < nkb; ++t) {
      const int64_t kk0 = static_cast<int64_t>(t) * kBK;
      if (t + 1 < nkb) st.fetch(h, ldh, d_in, kk0 + kBK, c0, tid);
      const f32x4 wv = *reinterpret_cast<const f32x4*>(wa + kk0 + 4 * q);
      const float d = va ? sa[kk0 / kGroup] : 0.0f;
      const float iv = inv_of(d);
      double a[4] = {err(wv.x, d, iv), err(wv.y, d, iv), err(wv.z, d, iv), err(wv.w, d, iv)};
      if (!va) a[0] = a[1] = a[2] = a[3] = 0.0;
      tile_mma(tile[t & 1], a, acc, lane);
      if (t + 1 < nkb) st.put(tile[(t + 1) & 1], tid);
      __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t col = c0 + 16 * c + j;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = rb + 4 * r + q;
        if (row < rows && col < d_in) {
          if (kStoreU) u[row * d_in + col] = acc[c][r];
          const float d = steps[row * G + col / kGroup];
          p[r] += acc[c][r] * err(w[row * d_in + col], d, inv_of(d));
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const double v = quarter_sum(p[r]);
    const int64_t row = rb + 4 * r + q;
    if (j == 0 && row < rows) part[row * n_split + blockIdx.y] = v;
  }
}

// obj[r] = sum_s part[r][s] in split order
__global__ __launch_bounds__(256) void part_sum_kernel(const double* __restrict__ part, int n_split, int64_t rows,
                                                       double* __restrict__ obj) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (r >= rows) return;
  double s = 0.0;
  for (int i = 0; i < n_split; ++i) s += part[r * n_split + i];
  obj[r] = s;
}

// Coordinate descent, kCdRows rows per workgroup (a wavefront per row), u = H e of each row in
// global memory (from joint_u_kernel).  The rows visit their groups in lockstep, so H_gg is staged
// once for all of them and the change u += H[:, g] d of every row that changed reads the 32 rows of
// H once (H symmetric: row g0 + i of H is column g0 + i).  Per group, each wavefront tries its
// row's candidates (on the fp64 matrix cores: H_gg times the changes of 16 candidates per
// product) and keeps the first minimum of dO (the current candidate has dO = 0 exactly).  Rows
// whose last sweep changed nothing stop sweeping (their trials would change nothing either); the
// workgroup runs until all have.
constexpr int kCdRows = 8;

__global__ __launch_bounds__(64 * kCdRows) void joint_cd_kernel(const float* __restrict__ w, int64_t d_in,
                                                                const float* __restrict__ h, int64_t ldh,
                                                                const float* __restrict__ alpha, int n_cand,
                                                                uint8_t* __restrict__ idx, float* __restrict__ steps,
                                                                double* __restrict__ u,
                                                                const double* __restrict__ part, int n_split,
                                                                int n_sweeps, double* __restrict__ obj_before,
                                                                double* __restrict__ obj_after,
                                                                int32_t* __restrict__ sweeps, int64_t rows) {
  constexpr int kThreads = 64 * kCdRows;
  __shared__ double hgg[kGroup][kGroup + 1];
  __shared__ double ug[kCdRows][kGroup], ecur[kCdRows][kGroup], dl[kCdRows][kGroup];
  __shared__ float wg[kCdRows][kGroup];
  __shared__ float cand[kCdRows][256];
  __shared__ double dobj[kCdRows][256];
  __shared__ int s_live, s_change;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kCdRows + wv;
  const bool have = row < rows;  // uniform per wavefront; rows past the end follow along unseen
  const int64_t rowc = have ? row : rows - 1;
  const int64_t G = d_in / kGroup;
  const float* wr = w + rowc * d_in;
  double* ur = u + rowc * d_in;
  uint8_t* ir = idx + rowc * G;
  if (have && lane == 0 && obj_before != nullptr) {
    double s = 0.0;
    for (int i = 0; i < n_split; ++i) s += part[row * n_split + i];
    obj_before[row] = s;
  }
  bool live = have;  // this row still sweeping (uniform per wavefront)
  int sw = 0;
  for (int sweep = 0; sweep < n_sweeps; ++sweep) {
    if (tid == 0) s_live = 0;
    __syncthreads();
    if (live && lane == 0) atomicOr(&s_live, 1 << wv);
    __syncthreads();
    if (s_live == 0) break;  // uniform
    if (live) ++sw;
    bool row_changed = false;
    // H_gg, w_g and the current index of group g + 1 are loaded during group g (they do not
    // change); u_g is read at the start of its group, after the previous group's update
    constexpr int kHPer = kGroup * kGroup / kThreads;
    float hpre[kHPer], wpre = 0.0f;
    int ipre = 0;
    auto prefetch = [&](int64_t gn) {
      const int64_t n0 = gn * kGroup;
#pragma unroll
      for (int p = 0; p < kHPer; ++p) {
        const int i = tid + p * kThreads;
        hpre[p] = h[(n0 + i / kGroup) * ldh + n0 + i % kGroup];
      }
      if (lane < kGroup) wpre = wr[n0 + lane];
      ipre = ir[gn];
    };
    prefetch(0);
    for (int64_t g = 0; g < G; ++g) {
      const int64_t g0 = g * kGroup;
#pragma unroll
      for (int p = 0; p < kHPer; ++p) {
        const int i = tid + p * kThreads;
        hgg[i / kGroup][i % kGroup] = static_cast<double>(hpre[p]);
      }
      if (lane < kGroup) {
        wg[wv][lane] = wpre;
        ug[wv][lane] = ur[g0 + lane];
      }
      const int kc = ipre < n_cand ? ipre : n_cand - 1;  // indices past the list: its last entry
      if (tid == 0) s_change = 0;
      __syncthreads();
      if (g + 1 < G) prefetch(g + 1);
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < kGroup; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(wg[wv][i]));
      for (int k = lane; k < n_cand; k += 64) cand[wv][k] = candidate(amax, alpha[k]);
      __syncthreads();
      if (lane < kGroup) {
        const float dc = cand[wv][kc];
        ecur[wv][lane] = err(wg[wv][lane], dc, inv_of(dc));
      }
      __syncthreads();
      if (live) {
        // 16 candidates at a time on the matrix cores: lane (q, j) supplies the change d of
        // candidate j at columns 16 kt + 4 q + s as the A operand, H_gg the B operand; the result
        // (H_gg d)[16 ct + j] of candidate 4 r + q (register r of tile ct) is dotted with
        // 2 u + H d by the same lane and summed over the 16 lanes of the quarter
        const int q = lane >> 4, j = lane & 15;
        for (int kb16 = 0; kb16 < n_cand; kb16 += 16) {
          const int ka = kb16 + j < n_cand ? kb16 + j : kc;
          const float da = cand[wv][ka], ia = inv_of(da);
          f64x4 hd[2] = {f64x4{0.0, 0.0, 0.0, 0.0}, f64x4{0.0, 0.0, 0.0, 0.0}};
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const int c = 16 * kt + 4 * q + s;
              const double a = err(wg[wv][c], da, ia) - ecur[wv][c];
#pragma unroll
              for (int ct = 0; ct < 2; ++ct)
                hd[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, hgg[c][16 * ct + j], hd[ct], 0, 0, 0);
            }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int k = kb16 + 4 * r + q;
            const float dk = cand[wv][k < n_cand ? k : kc];
            const float ik = inv_of(dk);
            double t = 0.0;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
              const int c = 16 * ct + j;
              const double dc = err(wg[wv][c], dk, ik) - ecur[wv][c];
              t += dc * (2.0 * ug[wv][c] + hd[ct][r]);
            }
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) t += __shfl_xor(t, off);
            if (j == 0 && k < n_cand) dobj[wv][k] = t;
          }
        }
      }
      __syncthreads();
      int kb = kc;
      if (live) {
        // first minimum: each lane scans its candidates lane, lane + 64, ... in order, then the
        // lanes combine, the lower index winning equal values
        double bv = __builtin_inf();
        int bi = 0x7FFFFFFF;
        for (int k = lane; k < n_cand; k += 64) {
          const double v = dobj[wv][k];
          if (v < bv || bi == 0x7FFFFFFF) {
            bv = v;
            bi = k;
          }
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const double ov = __shfl_xor(bv, off);
          const int oi = __shfl_xor(bi, off);
          if (ov < bv || (!(bv < ov) && oi < bi)) {
            bv = ov;
            bi = oi;
          }
        }
        kb = bi;
        if (lane == 0) {
          ir[g] = static_cast<uint8_t>(kb);
          if (kb != kc) atomicOr(&s_change, 1 << wv);
        }
        if (kb != kc) row_changed = true;
      }
      if (lane < kGroup) {
        const float db = cand[wv][kb];
        dl[wv][lane] = kb != kc ? err(wg[wv][lane], db, inv_of(db)) - ecur[wv][lane] : 0.0;
      }
      __syncthreads();
      // u += H[:, g] d for the rows that changed: kCols columns per thread at a time, H read once
      // for all rows, in two blocks of 16 of its 32 rows (the second block's loads in flight
      // across the first block's products)
      const int chg = s_change;  // uniform
      constexpr int kCols = 2, kIb = 16;
      if (chg != 0) {
        // wave-uniform row pointers and 32-bit lane offsets (global loads with a scalar base)
        double* ublk = u + static_cast<int64_t>(blockIdx.x) * kCdRows * d_in;
        for (int64_t j0 = 0; j0 < d_in; j0 += kCols * kThreads) {
          double a[kCols][kCdRows];
          float hv[2][kIb][kCols];
          uint32_t off[kCols];
          bool inb[kCols];
#pragma unroll
          for (int m = 0; m < kCols; ++m) {
            const int64_t jc = j0 + tid + m * kThreads;
            inb[m] = jc < d_in;
            off[m] = static_cast<uint32_t>(inb[m] ? jc : 0);
          }
          auto fetch = [&](int ib, int sl) {
#pragma unroll
            for (int ii = 0; ii < kIb; ++ii) {
              const float* hrow = h + (g0 + ib + ii) * ldh;
#pragma unroll
              for (int m = 0; m < kCols; ++m) hv[sl][ii][m] = hrow[off[m]];
            }
          };
          auto apply = [&](int ib, int sl) {
#pragma unroll
            for (int r = 0; r < kCdRows; ++r) {
              if ((chg >> r) & 1) {  // uniform
#pragma unroll
                for (int ii = 0; ii < kIb; ++ii) {
                  const double dr = dl[r][ib + ii];
#pragma unroll
                  for (int m = 0; m < kCols; ++m)
                    a[m][r] = __builtin_fma(static_cast<double>(hv[sl][ii][m]), dr, a[m][r]);
                }
              }
              asm volatile("" ::: "memory");  // one row's d at a time (bounds the live registers)
            }
          };
          fetch(0, 0);
#pragma unroll
          for (int r = 0; r < kCdRows; ++r) {
            const double* urow = ublk + r * d_in;
#pragma unroll
            for (int m = 0; m < kCols; ++m) a[m][r] = ((chg >> r) & 1) ? urow[off[m]] : 0.0;
          }
          fetch(kIb, 1);
          asm volatile("" ::: "memory");
          apply(0, 0);
          apply(kIb, 1);
#pragma unroll
          for (int r = 0; r < kCdRows; ++r) {
            double* urow = ublk + r * d_in;
#pragma unroll
            for (int m = 0; m < kCols; ++m)
              if (((chg >> r) & 1) && inb[m]) urow[off[m]] = a[m][r];
          }
        }
      }
      __syncthreads();
    }
    if (!row_changed) live = false;
  }
  // the steps of the result, then its objective e . u (u maintained through every change): a lane
  // per group, the lane partials summed in a fixed order
  if (!have) return;  // no barrier follows
  double s = 0.0;
  for (int64_t g = lane; g < G; g += 64) {
    float m = 0.0f;
    for (int i = 0; i < kGroup; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(wr[g * kGroup + i]));
    const float d = candidate(m, alpha[ir[g]]);
    steps[row * G + g] = d;
    const float inv = inv_of(d);
    for (int i = 0; i < kGroup; ++i) s += err(wr[g * kGroup + i], d, inv) * ur[g * kGroup + i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) {
    if (obj_after != nullptr) obj_after[row] = s;
    if (sweeps != nullptr) sweeps[row] = sw;
  }
}

inline unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

// column blocks per workgroup of the U kernel: enough workgroups to fill the chip
inline int split_cbs(int64_t rows, int64_t d_in) {
  const int64_t ncb = (d_in + kBN - 1) / kBN;
  const int64_t rblk = (rows + 63) / 64;
  int64_t want = (1024 + rblk - 1) / rblk;  // splits per row block
  if (want < 1) want = 1;
  if (want > ncb) want = ncb;
  return static_cast<int>((ncb + want - 1) / want);
}

}  // namespace
}  // namespace w4q

using namespace w4q;

int w4q_launch_pc_search(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
                         const float* alpha, int n_cand, float* scale, uint8_t* idx, float* obj,
                         float* obj_all, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(d_out));
#define W4Q_PC(NW)                                                                                         \
  hipLaunchKernelGGL(pc_search_kernel<NW>, grid, dim3(64 * NW), 0, s, w, d_in, h, ldh, alpha, n_cand, scale, \
                     idx, obj, obj_all)
  if (n_cand <= 16)
    W4Q_PC(1);
  else if (n_cand <= 32)
    W4Q_PC(2);
  else if (n_cand <= 48)
    W4Q_PC(3);
  else if (n_cand <= 64)
    W4Q_PC(4);
  else
    W4Q_PC(8);
#undef W4Q_PC
  return w4q_launch_status();
}

// bytes per row of the joint workspace: u (fp64 row) and the partial objectives
static int64_t joint_row_bytes(int64_t rows, int64_t d_in) {
  const int cbs = split_cbs(rows, d_in);
  const int64_t ncb = (d_in + kBN - 1) / kBN;
  const int64_t n_split = (ncb + cbs - 1) / cbs;
  return d_in * 8 + n_split * 8;
}

size_t w4q_joint_workspace(int64_t d_out, int64_t d_in) {
  const int64_t rows = d_out < 2048 ? d_out : 2048;  // rows per chunk; smaller workspaces run more chunks
  return static_cast<size_t>(rows * joint_row_bytes(rows, d_in));
}

// rows per chunk that ws_bytes holds (a multiple of 64, or all rows), 0 if fewer than 64
static int64_t joint_chunk_rows(int64_t d_out, int64_t d_in, size_t ws_bytes) {
  for (int64_t rows = d_out < 2048 ? d_out : 2048; rows > 0; rows = rows > 64 ? ((rows - 1) / 64) * 64 : 0)
    if (static_cast<size_t>(rows * joint_row_bytes(rows, d_in)) <= ws_bytes) return rows;
  return 0;
}

int w4q_launch_joint(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
                     const float* alpha, int n_cand, uint8_t* idx, float* steps, int n_sweeps,
                     double* obj_before, double* obj_after, int32_t* sweeps, void* ws, size_t ws_bytes,
                     hipStream_t s) {
  const int64_t G = d_in / kGroup;
  const int64_t chunk = joint_chunk_rows(d_out, d_in, ws_bytes);
  if (chunk == 0) return W4Q_EINVAL;
  if (alpha != nullptr) {  // steps from the indices (else the caller's steps are used as given)
    hipLaunchKernelGGL(steps_kernel, dim3(cdiv(d_out * G, 256)), dim3(256), 0, s, w, d_in, d_out, alpha, n_cand,
                       idx, steps);
    const int rc = w4q_launch_status();
    if (rc != W4Q_OK) return rc;
  }
  // one column split for every chunk: the one the workspace was sized with
  const int cbs = split_cbs(chunk, d_in);
  const int64_t ncb = (d_in + kBN - 1) / kBN;
  const int n_split = static_cast<int>((ncb + cbs - 1) / cbs);
  for (int64_t r0 = 0; r0 < d_out; r0 += chunk) {
    const int64_t rows = d_out - r0 < chunk ? d_out - r0 : chunk;
    double* u = static_cast<double*>(ws);
    double* part = u + rows * d_in;
    const dim3 grid(cdiv(rows, 64), static_cast<unsigned>(n_split));
    if (n_sweeps > 0) {
      hipLaunchKernelGGL(joint_u_kernel<true>, grid, dim3(256), 0, s, w + r0 * d_in, steps + r0 * G, rows, d_in,
                         h, ldh, cbs, u, part, n_split);
      int rc = w4q_launch_status();
      if (rc != W4Q_OK) return rc;
      hipLaunchKernelGGL(joint_cd_kernel, dim3(cdiv(rows, kCdRows)), dim3(64 * kCdRows), 0, s, w + r0 * d_in,
                         d_in, h, ldh, alpha, n_cand, idx + r0 * G, steps + r0 * G, u, part, n_split, n_sweeps,
                         obj_before ? obj_before + r0 : nullptr, obj_after ? obj_after + r0 : nullptr,
                         sweeps ? sweeps + r0 : nullptr, rows);
      rc = w4q_launch_status();
      if (rc != W4Q_OK) return rc;
    } else {  // the objective of the given steps only
      hipLaunchKernelGGL(joint_u_kernel<false>, grid, dim3(256), 0, s, w + r0 * d_in, steps + r0 * G, rows,
                         d_in, h, ldh, cbs, u, part, n_split);
      int rc = w4q_launch_status();
      if (rc != W4Q_OK) return rc;
      hipLaunchKernelGGL(part_sum_kernel, dim3(cdiv(rows, 256)), dim3(256), 0, s, part, n_split, rows,
                         obj_after + r0);
      rc = w4q_launch_status();
      if (rc != W4Q_OK) return rc;
    }
  }
  return W4Q_OK;
}

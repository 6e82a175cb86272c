// hessian.hip -- H = X^T X for bf16 calibration activations on the bf16 matrix cores.
//
// Method: blog "Opt.Gear-QAT: Preserving On-Device Performance with QAT", section 2 (the
// second-order output-reconstruction view from GPTQ; layer sensitivity from calibration
// inputs): for the objective of the model card's "Quantization Configuration",
// ||W X - Q(W) X||^2 is a quadratic form in the weight error with matrix X^T X.
//
// Only the tiles on and above the diagonal are computed (the algorithmic work is the unique
// entries of the symmetric result); each value is written to both (i, j) and (j, i), so H is
// bitwise symmetric.  X is row-major with the reduction (token) axis strided, while an MFMA
// fragment wants 8 consecutive tokens of one feature per lane: each thread loads an 8x8
// (tokens x features) bf16 block with 16-byte loads, transposes it in registers with byte
// permutes, and writes 8 feature rows of 8 tokens into LDS, where fragments are single
// 16-byte reads.  128x128 tiles, 4 wavefronts of 64x64 (2x2 v_mfma_f32_32x32x16_bf16
// blocks), 64 tokens per double-buffered LDS stage.
#include "common.hpp"

namespace w4q {
namespace {

constexpr int kThreads = 256;
constexpr int HT = 128;      // tile edge in features
constexpr int HK = 64;       // tokens per stage
constexpr int HLD = HK + 8;  // bf16 per LDS feature row (144 bytes)
constexpr int PD = 3;        // stages in flight between global memory and registers

__global__ __launch_bounds__(kThreads, 1) void hessian_kernel(const uint16_t* __restrict__ x, int64_t n_tok,
                                                              int64_t d, float* __restrict__ h,
                                                              int accumulate, int nt,
                                                              int64_t tiles, int64_t per_xcd) {
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][2 * HT * HLD];

  // workgroups are dealt to the 8 XCDs round-robin; each XCD takes a contiguous run of the
  // row-major upper-triangle tiles, so its resident tiles share I panels in its L2
  const int64_t t = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= tiles) return;
  // upper-triangle tile (ti <= tj) of this block
  int rem = static_cast<int>(t), ti = 0;
  while (rem >= nt - ti) {
    rem -= nt - ti;
    ++ti;
  }
  const int tj = ti + rem;
  const bool diag = ti == tj;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  // load role: 8 tokens (token block tb) x 8 features (feature block fb of the 256 staged)
  const int tb = lane & 7;
  const int fb = (lane >> 3) + 8 * wid;         // 0..31: 0..15 -> I rows, 16..31 -> J rows
  const bool jrow = fb >= 16;
  const int64_t feat = jrow ? (int64_t)tj * HT + 8 * (fb - 16) : (int64_t)ti * HT + 8 * fb;
  // (on a diagonal tile the J rows repeat the I rows; they are staged anyway, which keeps the
  // loads free of branches, but never read)
  // features past d read feature 0 instead (they only feed entries that are never stored);
  // tokens past n_tok read the last token and are zeroed when staged into LDS.  Unconditional
  // loads keep the prefetch ring free of branches and early waits.
  const uint16_t* xf = x + (feat < d ? feat : 0);

  struct Stage {
    u32x4 v[8];
  };
  Stage st[PD];
  auto gload = [&](int64_t k0, Stage& t) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      int64_t tok = k0 + 8 * tb + r;
      tok = tok < n_tok ? tok : n_tok - 1;
      t.v[r] = *reinterpret_cast<const u32x4*>(xf + tok * d);
    }
  };
  auto lstore = [&](int buf, int64_t k0, const Stage& t) {
    u32x4 rv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) rv[r] = (k0 + 8 * tb + r < n_tok) ? t.v[r] : u32x4{0u, 0u, 0u, 0u};
    // 8x8 transpose: out[f] holds tokens 0..7 of feature f as 4 bf16 pairs
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int wsel = f >> 1;
      const uint32_t sel = (f & 1) ? 0x07060302u : 0x05040100u;
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = rv[2 * p][wsel], hi = rv[2 * p + 1][wsel];
        o[p] = __builtin_amdgcn_perm(hi, lo, sel);
      }
      *reinterpret_cast<u32x4*>(&Xs[buf][(fb * 8 + f) * HLD + 8 * tb]) = u32x4{o[0], o[1], o[2], o[3]};
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // on a diagonal tile the (wm = 1, wn = 0) quadrant is the mirror of (0, 1): skip it
  const bool work = !(diag && wm == 1 && wn == 0);
  const int jbase = diag ? 0 : HT;  // B fragments come from the I rows on diagonal tiles
  const int fr = lane & 31;
  const int fk = 8 * (lane >> 5);
  const int64_t nstage = (n_tok + HK - 1) / HK;

  auto mma_stage = [&](int cur) {
    if (!work) return;
#pragma unroll
    for (int s = 0; s < HK / 16; ++s) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&Xs[cur][(wm * 64 + 32 * i + fr) * HLD + 16 * s + fk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Xs[cur][(jbase + wn * 64 + 32 * j + fr) * HLD + 16 * s + fk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // register ring PD stages deep: loads of stage st + PD - 1 are issued while stage st is
  // multiplied, and reach LDS one iteration before they are used
#pragma unroll
  for (int p = 0; p < PD - 1; ++p) gload(p * HK, st[p]);
  lstore(0, 0, st[0]);
  __syncthreads();
  for (int64_t s0 = 0; s0 < nstage; s0 += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const int64_t sg = s0 + u;
      if (sg >= nstage) break;  // uniform
      gload((sg + PD - 1) * HK, st[(u + PD - 1) % PD]);
      asm volatile("" ::: "memory");  // keep the prefetch issued here
      mma_stage(static_cast<int>(sg & 1));
      if (sg + 1 < nstage) lstore(static_cast<int>((sg + 1) & 1), (sg + 1) * HK, st[(u + 1) % PD]);
      __syncthreads();
    }
  }
  if (!work) return;

  // 32x32 accumulator layout: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, column l%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = (int64_t)tj * HT + wn * 64 + 32 * j + fr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = (int64_t)ti * HT + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= d || col >= d || row > col) continue;
        float v = acc[i][j][r];
        if (accumulate) v += h[row * d + col];
        h[row * d + col] = v;
        if (row != col) h[col * d + row] = v;
      }
    }
}

// ---------------------------------------------------------------------------------------
// 256x256 tiles for wide H (many tiles): 4 wavefronts of 128x128 (4x4 MFMA blocks, the
// accumulators live in AGPRs), 32 tokens per LDS stage, a 2-stage register prefetch ring.
// Per 16-token step a wavefront issues 16 MFMAs for 8 fragment reads (half the LDS traffic
// per MFMA of the 64x64 layout).  LDS rows are 32 tokens (64 bytes) with the 16-byte chunk c
// of row r stored at chunk c ^ ((r >> 1) & 3), so both the staging writes (4 lanes per row)
// and the fragment reads (8 consecutive rows per chunk) are bank-conflict free.
constexpr int BT = 256;    // tile edge in features
constexpr int BK = 32;     // tokens per stage
constexpr int BPD = 2;     // stages in flight between global memory and registers

__device__ __forceinline__ int swz32(int r, int c) { return r * 32 + 8 * (c ^ ((r >> 1) & 3)); }

__global__ __launch_bounds__(kThreads, 1) void hessian256_kernel(const uint16_t* __restrict__ x, int64_t n_tok,
                                                                 int64_t d, float* __restrict__ h,
                                                                 int accumulate, int nt,
                                                                 int64_t tiles, int64_t per_xcd) {
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][2 * BT * BK];

  const int64_t t = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= tiles) return;
  int rem = static_cast<int>(t), ti = 0;
  while (rem >= nt - ti) {
    rem -= nt - ti;
    ++ti;
  }
  const int tj = ti + rem;
  const bool diag = ti == tj;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  // load role: 8 tokens (token block tb of 4) x 8 features (feature block fb of 64 across the
  // 512 staged rows: 0..31 -> I rows, 32..63 -> J rows)
  const int tb = tid & 3;
  const int fb = tid >> 2;
  const bool jrow = fb >= 32;
  const int64_t feat = jrow ? (int64_t)tj * BT + 8 * (fb - 32) : (int64_t)ti * BT + 8 * fb;
  // features past d read feature 0 (they only feed entries that are never stored); tokens past
  // n_tok read the last token and are zeroed when staged
  const uint16_t* xf = x + (feat < d ? feat : 0);

  struct Stage {
    u32x4 v[8];
  };
  Stage st[BPD];
  auto gload = [&](int64_t k0, Stage& u) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      int64_t tok = k0 + 8 * tb + r;
      tok = tok < n_tok ? tok : n_tok - 1;
      u.v[r] = *reinterpret_cast<const u32x4*>(xf + tok * d);
    }
  };
  auto lstore = [&](int buf, int64_t k0, const Stage& u) {
    u32x4 rv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) rv[r] = (k0 + 8 * tb + r < n_tok) ? u.v[r] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int wsel = f >> 1;
      const uint32_t sel = (f & 1) ? 0x07060302u : 0x05040100u;
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) o[p] = __builtin_amdgcn_perm(rv[2 * p + 1][wsel], rv[2 * p][wsel], sel);
      *reinterpret_cast<u32x4*>(&Xs[buf][swz32(fb * 8 + f, tb)]) = u32x4{o[0], o[1], o[2], o[3]};
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const bool work = !(diag && wm == 1 && wn == 0);  // mirror quadrant of a diagonal tile
  const int jbase = diag ? 0 : BT;
  const int fr = lane & 31;
  const int fh = lane >> 5;
  const int64_t nstage = (n_tok + BK - 1) / BK;

  auto mma_stage = [&](int cur) {
    if (!work) return;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&Xs[cur][swz32(wm * 128 + 32 * i + fr, 2 * s + fh)]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Xs[cur][swz32(jbase + wn * 128 + 32 * j + fr, 2 * s + fh)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

#pragma unroll
  for (int p = 0; p < BPD - 1; ++p) gload(p * BK, st[p]);
  lstore(0, 0, st[0]);
  __syncthreads();
  for (int64_t s0 = 0; s0 < nstage; s0 += BPD) {
#pragma unroll
    for (int u = 0; u < BPD; ++u) {
      const int64_t sg = s0 + u;
      if (sg >= nstage) break;  // uniform
      gload((sg + BPD - 1) * BK, st[(u + BPD - 1) % BPD]);
      asm volatile("" ::: "memory");  // keep the prefetch issued here
      mma_stage(static_cast<int>(sg & 1));
      if (sg + 1 < nstage) lstore(static_cast<int>((sg + 1) & 1), (sg + 1) * BK, st[(u + 1) % BPD]);
      __syncthreads();
    }
  }
  if (!work) return;

  // 32x32 accumulator layout: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, column l%32
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = (int64_t)tj * BT + wn * 128 + 32 * j + fr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = (int64_t)ti * BT + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * fh + (r & 3);
        if (row >= d || col >= d || row > col) continue;
        float v = acc[i][j][r];
        if (accumulate) v += h[row * d + col];
        h[row * d + col] = v;
        if (row != col) h[col * d + row] = v;
      }
    }
}

}  // namespace
}  // namespace w4q

using namespace w4q;

int w4q_launch_hessian(const uint16_t* x, int64_t n_tok, int64_t d, float* h, int accumulate,
                       hipStream_t s) {
  // 256-wide tiles when they still give at least one tile per compute unit
  const int64_t nt2 = (d + BT - 1) / BT;
  const int64_t tiles2 = nt2 * (nt2 + 1) / 2;
  if (tiles2 >= 256) {
    const int64_t per2 = (tiles2 + 7) / 8;
    if (8 * per2 > 0x7FFFFFFF) return W4Q_EUNSUPPORTED;
    hipLaunchKernelGGL(hessian256_kernel, dim3(static_cast<unsigned>(8 * per2)), dim3(kThreads), 0, s, x,
                       n_tok, d, h, accumulate, static_cast<int>(nt2), tiles2, per2);
    return w4q_launch_status();
  }
  const int64_t nt = (d + HT - 1) / HT;
  const int64_t tiles = nt * (nt + 1) / 2;
  const int64_t per_xcd = (tiles + 7) / 8;
  if (8 * per_xcd > 0x7FFFFFFF) return W4Q_EUNSUPPORTED;
  hipLaunchKernelGGL(hessian_kernel, dim3(static_cast<unsigned>(8 * per_xcd)), dim3(kThreads), 0, s, x,
                     n_tok, d, h, accumulate, static_cast<int>(nt), tiles, per_xcd);
  return w4q_launch_status();
}

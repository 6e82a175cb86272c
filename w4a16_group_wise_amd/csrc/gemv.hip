// gemv.hip -- W4A16 product for a few activation rows (decode): streams the packed INT4 codes
// and fp16 scales from HBM once and keeps the activations in registers.
//
// Method: model card "Opt.Gear-1B-qat-int4-per-channel-unquantized" (W4A16: INT4 weights with
// 16-bit activations; weight memory and bandwidth set the speed) with the group-32 symmetric
// grid of blog "Opt.Gear-QAT: Preserving On-Device Performance with QAT".
//   y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] * q[n][k]
//
// Mapping: a group of 32 codes is one 16-byte load, so a lane owns one group column; LPR lanes
// (a power of two dividing G) cover one row per chunk of LPR groups, and a wavefront works on
// 64 / LPR rows at once, RS row-steps deep, walking the chunks along d_in.  Loads of a row are
// contiguous (LPR * 16 bytes).  The lane keeps its group's activations as bf16 pairs in
// registers, reused for all the rows of the wavefront.
//
// Dequantisation in registers: the nibble n = q + 8 goes into the top four mantissa bits of a
// bf16 with exponent 2^7, giving the exact value 8 * (24 + q); v_dot2 multiplies two such codes
// with two activations into an fp32 sum.  The constant part is removed per group by the same
// dot2 chain run on the code q = 0 (bitwise the same sum when every code of the group is 0),
// and the factor 8 is folded into the scale.  The bias is 24/|q| times the signal, so the
// fp32 sum error stays near 2^-24 * 31 * sum|x| per group.
#include "common.hpp"

namespace w4q {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair with exponent 2^7, zero mantissa
constexpr uint32_t kMask = 0x00780078u;   // mantissa bits 3..6 of each half
constexpr uint32_t kZero = 0x43404340u;   // code q = 0 (n = 8) in both halves

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

// 8 activations x[8b .. 8b+7] as 4 dwords (x0,x1)(x2,x3)(x4,x5)(x6,x7) -> the pairs
// (x0,x4)(x1,x5)(x2,x6)(x3,x7) that match the nibble pairs extracted below.
__device__ __forceinline__ void pair_x(const u32x4 d, uint32_t (&p)[4]) {
  p[0] = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);
  p[1] = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);
  p[2] = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);
  p[3] = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);
}

// 8 two's-complement nibbles -> biased bf16 code pairs (nibble i and i+4 share a dword).
__device__ __forceinline__ void codes_bf16(uint32_t v, uint32_t (&c)[4]) {
  v ^= 0x88888888u;  // two's complement -> offset binary n = q + 8
  c[0] = ((v << 3) & kMask) | kMagic;
  c[1] = ((v >> 1) & kMask) | kMagic;
  c[2] = ((v >> 5) & kMask) | kMagic;
  c[3] = ((v >> 9) & kMask) | kMagic;
}

template <int MT, int LPR, int RS>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint16_t* __restrict__ x, int64_t m_rows,
                                                        const uint8_t* __restrict__ packed,
                                                        const uint16_t* __restrict__ s16,
                                                        int64_t d_out, int64_t d_in,
                                                        void* __restrict__ y, int y_dtype) {
  constexpr int RPS = 64 / LPR;  // rows per row-step
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;
  const int j = lane % LPR;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
  const int64_t row0 = wave * (RPS * RS);
  if (row0 >= d_out) return;  // uniform per wavefront
  const int64_t G = d_in / kGroup;
  const int64_t nchunk = G / LPR;
  const int64_t prow = d_in / 2;

  float acc[RS][MT];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[rs][m] = 0.0f;

  for (int64_t c = 0; c < nchunk; ++c) {
    const int64_t g = c * LPR + j;
    // codes + scales of this chunk for all row-steps (issued first, HBM stream)
    u32x4 cw[RS];
    float sc[RS];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      const int64_t n = row0 + rs * RPS + sub;
      const bool ok = n < d_out;
      const int64_t nn = ok ? n : 0;
      cw[rs] = *reinterpret_cast<const u32x4*>(packed + nn * prow + g * 16);
      sc[rs] = ok ? f16_bits_to_f32(s16[nn * G + g]) * 0.125f : 0.0f;
    }
    // activations of this group, paired, plus the zero-code sum
    uint32_t xp[MT][16];
    float corr[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const bool okm = m < m_rows;
      const uint16_t* xr = x + (okm ? m : 0) * d_in + g * kGroup;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        u32x4 d = *reinterpret_cast<const u32x4*>(xr + 8 * b);
        if (!okm) d = u32x4{0u, 0u, 0u, 0u};
        uint32_t p[4];
        pair_x(d, p);
#pragma unroll
        for (int i = 0; i < 4; ++i) xp[m][4 * b + i] = p[i];
      }
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) a = dot2(xp[m][i], kZero, a);
      corr[m] = a;
    }
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      uint32_t cb[16];
      const uint32_t words[4] = {cw[rs].x, cw[rs].y, cw[rs].z, cw[rs].w};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint32_t cc[4];
        codes_bf16(words[b], cc);
#pragma unroll
        for (int i = 0; i < 4; ++i) cb[4 * b + i] = cc[i];
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a = dot2(xp[m][i], cb[i], a);
        acc[rs][m] = __builtin_fmaf(sc[rs], a - corr[m], acc[rs][m]);
      }
    }
  }
  // reduce the LPR lane partials of each row (fixed butterfly order)
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const int64_t n = row0 + rs * RPS + sub;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[rs][m];
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      if (j == 0 && n < d_out && m < m_rows) {
        if (y_dtype == 0)
          reinterpret_cast<float*>(y)[m * d_out + n] = v;
        else
          reinterpret_cast<uint16_t*>(y)[m * d_out + n] = f32_to_bf16_bits(v);
      }
    }
  }
}

template <int MT, int LPR>
int launch_lpr(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
               int64_t d_out, int64_t d_in, void* y, int ydt, hipStream_t s) {
  constexpr int RPS = 64 / LPR;
  const int64_t waves1 = (d_out + RPS - 1) / RPS;
  // deeper row-steps amortise the activation loads; keep >= ~1024 wavefronts in flight
  if (waves1 >= 4 * 1024) {
    const int64_t waves = (d_out + 4 * RPS - 1) / (4 * RPS);
    hipLaunchKernelGGL((gemv_kernel<MT, LPR, 4>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                       dim3(kThreads), 0, s, x, m, packed, s16, d_out, d_in, y, ydt);
  } else if (waves1 >= 2 * 1024) {
    const int64_t waves = (d_out + 2 * RPS - 1) / (2 * RPS);
    hipLaunchKernelGGL((gemv_kernel<MT, LPR, 2>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                       dim3(kThreads), 0, s, x, m, packed, s16, d_out, d_in, y, ydt);
  } else {
    hipLaunchKernelGGL((gemv_kernel<MT, LPR, 1>), dim3(static_cast<unsigned>((waves1 + 3) / 4)),
                       dim3(kThreads), 0, s, x, m, packed, s16, d_out, d_in, y, ydt);
  }
  return w4q_launch_status();
}

template <int MT>
int launch_mt(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
              int64_t d_out, int64_t d_in, void* y, int ydt, hipStream_t s) {
  const int64_t G = d_in / kGroup;
  if (G % 64 == 0) return launch_lpr<MT, 64>(x, m, packed, s16, d_out, d_in, y, ydt, s);
  if (G % 32 == 0) return launch_lpr<MT, 32>(x, m, packed, s16, d_out, d_in, y, ydt, s);
  if (G % 16 == 0) return launch_lpr<MT, 16>(x, m, packed, s16, d_out, d_in, y, ydt, s);
  if (G % 8 == 0) return launch_lpr<MT, 8>(x, m, packed, s16, d_out, d_in, y, ydt, s);
  if (G % 4 == 0) return launch_lpr<MT, 4>(x, m, packed, s16, d_out, d_in, y, ydt, s);
  if (G % 2 == 0) return launch_lpr<MT, 2>(x, m, packed, s16, d_out, d_in, y, ydt, s);
  return launch_lpr<MT, 1>(x, m, packed, s16, d_out, d_in, y, ydt, s);
}

}  // namespace
}  // namespace w4q

using namespace w4q;

// Activation rows are processed four at a time; each slice of rows re-streams the weights.
int w4q_launch_gemv(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                    int64_t d_out, int64_t d_in, void* y, int y_dtype, hipStream_t s) {
  const size_t ysz = y_dtype == 0 ? 4 : 2;
  for (int64_t m0 = 0; m0 < m; m0 += 4) {
    const int64_t mt = (m - m0) < 4 ? (m - m0) : 4;
    const uint16_t* xs = x + m0 * d_in;
    void* ys = static_cast<char*>(y) + static_cast<size_t>(m0 * d_out) * ysz;
    int rc;
    if (mt == 1)
      rc = launch_mt<1>(xs, mt, packed, s16, d_out, d_in, ys, y_dtype, s);
    else if (mt == 2)
      rc = launch_mt<2>(xs, mt, packed, s16, d_out, d_in, ys, y_dtype, s);
    else
      rc = launch_mt<4>(xs, mt, packed, s16, d_out, d_in, ys, y_dtype, s);
    if (rc != W4Q_OK) return rc;
  }
  return W4Q_OK;
}

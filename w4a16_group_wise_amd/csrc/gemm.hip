// gemm.hip -- W4A16 product for many activation rows (prefill) on the bf16 matrix cores.
//
// Method: model card "Opt.Gear-1B-qat-int4-per-channel-unquantized" (W4A16 deployment) with
// the group-32 symmetric grid of blog "Opt.Gear-QAT: Preserving On-Device Performance with
// QAT":   y[m][n] = sum_g s[n][g] * P_g[m][n],   P_g[m][n] = sum_{k in g} x[m][k] * q[n][k].
//
// Each K-step is exactly one group of 32.  The codes are expanded to bf16 in registers
// (exact: small integers) and staged with the activation tile in LDS; two
// v_mfma_f32_32x32x16_bf16 per 32x32 block form P_g from a zero accumulator, and the fp32
// scale of column n is applied once per group (acc += s * P_g), so the weights enter the
// products unrounded.
//
// Tiling: 128x128 block tile, 4 wavefronts of 64x64 (2x2 MFMA blocks each), double-buffered
// LDS with one barrier per group, and a register ring that keeps the global loads of the next
// PD - 1 groups in flight (one group of compute is far shorter than a memory round trip).
// LDS rows are padded to 80 bytes so the 16-byte fragment reads of 8 consecutive lanes fall
// in distinct banks.
#include "common.hpp"

namespace w4q {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int LDA = 40;  // bf16 per LDS row (32 + 8 pad)
constexpr int PD = 4;    // groups in flight between global memory and registers

// 16 two's-complement nibbles (k ascending) -> 16 exact bf16 codes as 8 dwords.
__device__ __forceinline__ void expand16(u32x2 v, u32x4& lo, u32x4& hi) {
  uint32_t o[8];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t word = w == 0 ? v.x : v.y;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int q0 = static_cast<int>(word << (28 - 8 * p)) >> 28;
      const int q1 = static_cast<int>(word << (24 - 8 * p)) >> 28;
      const uint32_t f0 = __builtin_bit_cast(uint32_t, static_cast<float>(q0));
      const uint32_t f1 = __builtin_bit_cast(uint32_t, static_cast<float>(q1));
      o[4 * w + p] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);  // small integers: exact
    }
  }
  lo = u32x4{o[0], o[1], o[2], o[3]};
  hi = u32x4{o[4], o[5], o[6], o[7]};
}

__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                           const uint8_t* __restrict__ packed,
                                                           const uint16_t* __restrict__ s16,
                                                           int64_t N, int64_t K,
                                                           void* __restrict__ y, int y_dtype) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDA];
  __shared__ float Ss[2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t G = K / kGroup;
  const int64_t prow = K / 2;

  // load roles: A row ar (two 16-byte halves by ah), B column bc (8 bytes = 16 codes by bh)
  const int ar = tid >> 1, ah = tid & 1;
  const int bc = tid >> 1, bh = tid & 1;
  // rows / columns past the edge read row / column 0 instead: they only feed outputs that
  // are never stored, and unconditional loads keep the prefetch free of branches and waits
  const int64_t arow = m0 + ar < M ? m0 + ar : 0;
  const int64_t bcol = n0 + bc < N ? n0 + bc : 0;
  const uint16_t* xa = x + arow * K + 16 * ah;
  const uint8_t* pb = packed + bcol * prow + 8 * bh;
  const uint16_t* sb = s16 + bcol * G;

  // global -> register ring, PD groups deep: the loads of group g + PD - 1 are issued while
  // group g is multiplied, and reach LDS one iteration before they are used
  struct Stage {
    u32x4 a0, a1;
    u32x2 b;
    uint32_t sc;
  };
  Stage st[PD];
  auto gload = [&](int64_t g, Stage& t) {
    const int64_t gg = g < G ? g : G - 1;  // clamped: the tail re-reads the last group
    t.a0 = *reinterpret_cast<const u32x4*>(xa + gg * kGroup);
    t.a1 = *reinterpret_cast<const u32x4*>(xa + gg * kGroup + 8);
    t.b = *reinterpret_cast<const u32x2*>(pb + gg * 16);
    t.sc = sb[gg];
  };
  auto lstore = [&](int buf, const Stage& t) {
    *reinterpret_cast<u32x4*>(&As[buf][ar * LDA + 16 * ah]) = t.a0;
    *reinterpret_cast<u32x4*>(&As[buf][ar * LDA + 16 * ah + 8]) = t.a1;
    u32x4 blo, bhi;
    expand16(t.b, blo, bhi);
    *reinterpret_cast<u32x4*>(&Bs[buf][bc * LDA + 16 * bh]) = blo;
    *reinterpret_cast<u32x4*>(&Bs[buf][bc * LDA + 16 * bh + 8]) = bhi;
    if (bh == 0) Ss[buf][bc] = f16_bits_to_f32(static_cast<uint16_t>(t.sc));
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const f32x16 zero16 = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f,
                         0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  const int fr = lane & 31;
  const int fk = 8 * (lane >> 5);
  auto mma_group = [&](int cur) {
    f32x16 tmp[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[cur][(wm * 64 + 32 * i + fr) * LDA + 16 * s + fk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][(wn * 64 + 32 * j + fr) * LDA + 16 * s + fk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          tmp[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], s == 0 ? zero16 : tmp[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float sc = Ss[cur][wn * 64 + 32 * j + fr];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(sc, tmp[i][j][r], acc[i][j][r]);
    }
  };

#pragma unroll
  for (int p = 0; p < PD - 1; ++p) gload(p, st[p]);
  lstore(0, st[0]);
  __syncthreads();
  for (int64_t g0 = 0; g0 < G; g0 += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const int64_t g = g0 + u;
      if (g >= G) break;  // uniform
      gload(g + PD - 1, st[(u + PD - 1) % PD]);
      asm volatile("" ::: "memory");  // keep the prefetch issued here
      mma_group(static_cast<int>(g & 1));
      if (g + 1 < G) lstore(static_cast<int>((g + 1) & 1), st[(u + 1) % PD]);
      __syncthreads();
    }
  }

  // 32x32 accumulator layout: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, column l%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + 32 * j + fr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) {
          if (y_dtype == 0)
            reinterpret_cast<float*>(y)[row * N + col] = acc[i][j][r];
          else
            reinterpret_cast<uint16_t*>(y)[row * N + col] = f32_to_bf16_bits(acc[i][j][r]);
        }
      }
    }
}

}  // namespace
}  // namespace w4q

using namespace w4q;

int w4q_launch_gemm(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                    int64_t d_out, int64_t d_in, void* y, int y_dtype, hipStream_t s) {
  const int64_t gm = (m + BM - 1) / BM, gn = (d_out + BN - 1) / BN;
  if (gm > 65535 || gn > 0x7FFFFFFF) return W4Q_EUNSUPPORTED;
  hipLaunchKernelGGL(gemm_kernel, dim3(static_cast<unsigned>(gn), static_cast<unsigned>(gm)),
                     dim3(kThreads), 0, s, x, m, packed, s16, d_out, d_in, y, y_dtype);
  return w4q_launch_status();
}

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
// Tiling: 256x128 (or 128x128 for short M) block tile, wavefronts of 64x64 (2x2 MFMA blocks
// each) that all share one expansion of the codes per group, double-buffered LDS with one
// barrier per group, and a register ring that keeps the global loads of the next PD - 1
// groups in flight (one group of compute is far shorter than a memory round trip).  LDS rows
// are XOR-swizzled in 16-byte chunks so fragment reads and tile writes are bank-conflict free.
#include "common.hpp"

namespace w4q {
namespace {

constexpr int WN = 2;   // wavefronts along N (64 columns each)
constexpr int BN = 64 * WN;
constexpr int PD = 4;   // groups in flight between global memory and registers

// LDS tiles are rows of 32 bf16 (4 chunks of 16 bytes, no padding); chunk c of row r is stored
// at chunk c ^ ((r >> 1) & 3).  Eight lanes reading one chunk of eight consecutive rows, and
// eight lanes writing the four chunks of two consecutive rows, then hit distinct banks.
__device__ __forceinline__ int swz(int r, int c) { return r * 32 + 8 * (c ^ ((r >> 1) & 3)); }

// 8 two's-complement nibbles (k ascending) -> 8 exact bf16 codes as 4 dwords.
__device__ __forceinline__ u32x4 expand8(uint32_t word) {
  uint32_t o[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int q0 = static_cast<int>(word << (28 - 8 * p)) >> 28;
    const int q1 = static_cast<int>(word << (24 - 8 * p)) >> 28;
    const uint32_t f0 = __builtin_bit_cast(uint32_t, static_cast<float>(q0));
    const uint32_t f1 = __builtin_bit_cast(uint32_t, static_cast<float>(q1));
    o[p] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);  // small integers: exact in bf16
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}

// WM wavefronts along M (64 rows each) x WN along N; block tile (64 WM) x 128.
template <int WM>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                          const uint8_t* __restrict__ packed,
                                                          const uint16_t* __restrict__ s16,
                                                          int64_t N, int64_t K,
                                                          void* __restrict__ y, int y_dtype,
                                                          int64_t gn, int64_t tiles, int64_t per_xcd) {
  constexpr int NT = 64 * WM * WN;  // threads
  constexpr int BM = 64 * WM;
  constexpr int BJ = BN * 4 / NT;   // B dwords (8 codes) per thread per group
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * 32];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * 32];
  __shared__ float Ss[2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid % WM, wn = wid / WM;
  // workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous run of tiles in
  // N-fastest order, so the tiles resident on one XCD share their activation panel in its L2
  const int64_t t = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= tiles) return;
  const int64_t m0 = (t / gn) * BM;
  const int64_t n0 = (t % gn) * BN;
  const int G = static_cast<int>(K / kGroup);
  const int64_t prow = K / 2;

  // load roles.  A: row tid/2, 16-byte chunks 2*(tid%2) and +1.  B: column (tid + NT*j)/4,
  // dword (tid % 4) = codes 8*(tid%4) .. +7.  Rows / columns past the edge read row / column 0
  // (they only feed outputs that are never stored), so every load is unconditional.
  const int ar = tid >> 1, ac = 2 * (tid & 1);
  const uint16_t* xa = x + (m0 + ar < M ? m0 + ar : 0) * K + 8 * ac;
  const uint32_t* pb[BJ];
  int bcol[BJ];
#pragma unroll
  for (int j = 0; j < BJ; ++j) {
    bcol[j] = (tid + NT * j) >> 2;
    const int64_t n = n0 + bcol[j] < N ? n0 + bcol[j] : 0;
    pb[j] = reinterpret_cast<const uint32_t*>(packed + n * prow) + (tid & 3);
  }
  const bool s_role = tid < BN;
  const uint16_t* sb = s16 + (s_role && n0 + tid < N ? n0 + tid : 0) * G;

  struct Stage {
    u32x4 a0, a1;
    uint32_t b[BJ];
    uint32_t sc;
  };
  Stage st[PD];
  auto gload = [&](int g, Stage& t) {
    const int gg = g < G ? g : G - 1;  // clamped: the tail re-reads the last group
    t.a0 = *reinterpret_cast<const u32x4*>(xa + gg * kGroup);
    t.a1 = *reinterpret_cast<const u32x4*>(xa + gg * kGroup + 8);
#pragma unroll
    for (int j = 0; j < BJ; ++j) t.b[j] = pb[j][gg * 4];
    t.sc = sb[gg];
  };
  auto lstore = [&](int buf, const Stage& t) {
    *reinterpret_cast<u32x4*>(&As[buf][swz(ar, ac)]) = t.a0;
    *reinterpret_cast<u32x4*>(&As[buf][swz(ar, ac + 1)]) = t.a1;
#pragma unroll
    for (int j = 0; j < BJ; ++j)
      *reinterpret_cast<u32x4*>(&Bs[buf][swz(bcol[j], tid & 3)]) = expand8(t.b[j]);
    if (s_role) Ss[buf][tid] = f16_bits_to_f32(static_cast<uint16_t>(t.sc));
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
  const int fh = lane >> 5;
  auto mma_group = [&](int cur) {
    f32x16 tmp[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[cur][swz(wm * 64 + 32 * i + fr, 2 * s + fh)]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][swz(wn * 64 + 32 * j + fr, 2 * s + fh)]);
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
  for (int g0 = 0; g0 < G; g0 += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const int g = g0 + u;
      if (g >= G) break;  // uniform
      gload(g + PD - 1, st[(u + PD - 1) % PD]);
      asm volatile("" ::: "memory");  // keep the prefetch issued here
      mma_group(g & 1);
      if (g + 1 < G) lstore((g + 1) & 1, st[(u + 1) % PD]);
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
        const int64_t row = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * fh + (r & 3);
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
  if (d_in / kGroup > 0x7FFFFFFF) return W4Q_EUNSUPPORTED;
  const int64_t gn = (d_out + BN - 1) / BN;
  // 256-row tiles (8 wavefronts share one expansion of the codes) when they still give at
  // least one tile per compute unit, 128-row tiles otherwise
  const int64_t gm4 = (m + 255) / 256, gm2 = (m + 127) / 128;
  const bool big = gm4 * gn >= 256;
  const int64_t tiles = (big ? gm4 : gm2) * gn;
  const int64_t per_xcd = (tiles + 7) / 8;
  if (8 * per_xcd > 0x7FFFFFFF) return W4Q_EUNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(8 * per_xcd));
  if (big)
    hipLaunchKernelGGL(gemm_kernel<4>, grid, dim3(64 * 4 * WN), 0, s, x, m, packed, s16, d_out, d_in, y,
                       y_dtype, gn, tiles, per_xcd);
  else
    hipLaunchKernelGGL(gemm_kernel<2>, grid, dim3(64 * 2 * WN), 0, s, x, m, packed, s16, d_out, d_in, y,
                       y_dtype, gn, tiles, per_xcd);
  return w4q_launch_status();
}

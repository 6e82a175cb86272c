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
// Where this kernel would have fewer tiles than compute units, the exact product runs instead
// on the stream-K kernel further down, with each weight split into two bf16-exact parts.
#include "common.hpp"

namespace w4q {
namespace {

constexpr int WN = 2;   // wavefronts along N (64 columns each)
constexpr int BN = 64 * WN;
constexpr int PD = 4;   // groups in flight between global memory and registers

// LDS tiles are rows of 32 bf16 (4 chunks of 16 bytes, no padding); chunk c of row r is stored
// at chunk c ^ swz_f(r).  Measured on gfx950: a 16-byte LDS read is served in passes of 16
// lanes -- in each half of the wavefront, the four lane quads whose index (lane bits 2..4) has
// even parity form one pass and the other four the second -- and a 16-byte LDS write in passes of
// 8 consecutive lanes (128 bytes).  swz_f(r) = (r1 ^ r4) | r2 << 1 (r_i: bit i of r) is
// one-to-one on the quads of each parity class (fragment reads: lane l reads row l % 32) and on
// bits 1..2 of r (writes of consecutive rows or columns), so every pass of the fragment reads
// and of the tile writes below hits distinct 16-byte bank slots.
__device__ __forceinline__ int swz_f(int r) { return (((r >> 1) ^ (r >> 4)) & 1) | ((r >> 1) & 2); }
__device__ __forceinline__ int swz(int r, int c) { return r * 32 + 8 * (c ^ swz_f(r)); }

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
__global__ __launch_bounds__(64 * WM * WN) void gemm_group_kernel(const uint16_t* __restrict__ x, int64_t M,
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


// ---------------------------------------------------------------------------------------
// Matrix-core kernel: 256x256 output tiles, 8 wavefronts (two per SIMD) of 256x32 (8 blocks of
// v_mfma_f32_32x32x16_bf16 down the rows), one K-group (32 codes) per stage, two wavefronts per
// SIMD.  Each wavefront owns 32 whole columns, so every code is dequantized exactly once (about
// three vector instructions per code; with the vector work removed the kernel is only about
// 11 % faster).
//   x tile   : buffer loads straight to LDS, [row][16-byte chunk] with chunk c of row r at
//              position c ^ swz_f(r), 5 stage buffers (loads run 4 stages ahead); each
//              wavefront loads 32 rows and reads its A fragments from there.
//   codes    : 16 bytes (the group's 32 nibbles) per column, loaded to LDS by wavefronts 0-3;
//              fp16 scales 16 bytes (8 groups) per column every 8 groups, by wavefronts 4-7.
//   weights  : never stored: each lane reads the code words of its B fragment (one 32-bit word,
//              8 codes, per step) and its column's scale from LDS and forms the bf16 fragment
//              in registers, one step ahead of the products.  (LDS writes are the
//              scarce resource on gfx950 -- about a third of the read bandwidth -- so only the
//              activations go through LDS as bf16.)
// The weights are dequantized to bf16, w = bf16_RNE(s * q) (w4a16_gemm_dq), or split into two
// exact bf16 parts (w4a16_gemm below 256 tiles of the per-group kernel; see kSplit).
// Work split as for the Hessian: stream-K over (tile, group), partial tiles summed in a fixed
// order by a second kernel.  All global loads are the asm loads to LDS, so the explicit vmcnt
// waits count exactly 3 loads per stage and wavefront (2 x rows, 1 codes or scales or empty).
constexpr int GT = 256;                // tile edge (x rows and output columns)
constexpr int GNB = 5;                 // x / codes stage buffers (loads run 4 stages ahead)
constexpr int kGThreads = 512;
constexpr int kXStage = GT * 32 * 2;   // 16 KB
constexpr int kCStage = GT * 16;       // 4 KB
constexpr int kSBlock = GT * 16;       // 4 KB: scales of 8 groups
constexpr int kGTileElems = GT * GT;
constexpr int kGMinChunk = 16;
constexpr int kGMaxBlocks = 256;
constexpr int kOpsPerStage = 3;
constexpr int kOffC = GNB * kXStage;                // 80 KB
constexpr int kOffS = kOffC + GNB * kCStage;        // 100 KB
constexpr int kOffJunk = kOffS + 2 * kSBlock;       // 108 KB (target of the empty loads)
constexpr int kGemmLds = kOffJunk + 1024;           // 109 KB

// byte offset of 16-byte chunk c within LDS row r (64-byte rows): position c ^ swz_f(r) (the
// fragment reads are then free of bank conflicts)
__device__ __forceinline__ int gswz(int r, int c) { return 16 * (c ^ swz_f(r)); }

// partial-tile layout of the accumulators: wavefront w, block i, 16-byte quarter a, lane; 1 KB
// per store instruction
__device__ __forceinline__ int64_t gpart_off(int w, int i, int a, int lane) {
  return (int64_t)(((w * 8 + i) * 4 + a) * 256 + 4 * lane);
}

// Store one 32x32 accumulator block (rows row0.., columns col0..) of y.
__device__ __forceinline__ void gstore_block(void* __restrict__ y, int y_dtype, int M, int N, int row0, int col0,
                                             const f32x16& v, int lane) {
  const int col = col0 + (lane & 31);
  if (col >= N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = row0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (row >= M) continue;
    const int64_t o = (int64_t)row * N + col;
    if (y_dtype == 0)
      reinterpret_cast<float*>(y)[o] = v[r];
    else
      reinterpret_cast<uint16_t*>(y)[o] = f32_to_bf16_bits(v[r]);
  }
}

// kSplit: exact weights.  s * q is formed as two bf16 parts, s_hi * q and s_lo * q, with s_hi = s
// rounded to 5 significant bits and s_lo = s - s_hi (at most 5 significant bits too, since
// |s - s_hi| <= 32 units of s's 11-bit significand): each part times a code (at most 3
// significant bits) fits bf16's 8 bits exactly, so the two products per weight enter the fp32
// sums unrounded.  Otherwise the weights are dequantized to bf16: w = bf16_RNE(s * q).
template <bool kSplit>
__global__ __launch_bounds__(kGThreads, 1) void gemm_dq_kernel(const uint16_t* __restrict__ x, int M,
                                                                const uint8_t* __restrict__ packed,
                                                                const uint16_t* __restrict__ s16, int N, int K,
                                                                void* __restrict__ y, int y_dtype, int tn_count,
                                                                int total, int chunk, int nblk, int per_xcd,
                                                                float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kGemmLds];
  const int G = K >> 5;
  const int lb = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lb >= nblk) return;
  const int it_begin = lb * chunk;
  const int it_end = it_begin + chunk < total ? it_begin + chunk : total;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = lds_addr(lds);

  // x loads: load q (0..1) of wave w fills rows 32 w + 16 q .. + 15, lane l -> row + l / 4,
  // position l % 4, which holds chunk (l % 4) ^ swz_f(row)
  int xvo[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 32 * wid + 16 * q + (lane >> 2);
    xvo[q] = r * K * 2 + 16 * ((lane & 3) ^ swz_f(r));
  }
  // codes (waves 0-3) or scales (waves 4-7): column 64 (w % 4) + l of the tile
  const int lcol = 64 * (wid & 3) + lane;
  const int cvo = lcol * (K >> 1);
  const int svo = lcol * G * 2;

  // fragment reads: lane l reads row (col) base + l % 32, chunk 2 kk + l / 32
  const int fr = lane & 31, fh = lane >> 5;

  const f32x16 zero16 = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f,
                         0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};

  int it = it_begin;
  while (it < it_end) {
    const int t = it / G;
    const int s0 = it - t * G;
    const int s1 = s0 + (it_end - it) < G ? s0 + (it_end - it) : G;
    const int tm = t / tn_count, tn = t - tm * tn_count;
    const int m0 = tm * GT, n0 = tn * GT;
    const uint16_t* xt = x + (int64_t)m0 * K;
    const uint8_t* pt = packed + (int64_t)n0 * (K >> 1);
    const uint16_t* st = s16 + (int64_t)n0 * G;
    const int xbytes = (M - m0) * K * 2;
    const int cbytes = (N - n0) * (K >> 1);
    const int sbytes = (N - n0) * G * 2;

    // stage buffer of group g + k (0 <= k < GNB) from gb = g % GNB
    auto sbuf = [](int gb, int k) { return gb + k >= GNB ? gb + k - GNB : gb + k; };
    // loads of group g into stage buffer b: x rows; codes (waves 0-3) or, when g starts a block
    // of 8 or the range, scales (waves 4-7; otherwise an empty load to the junk area)
    auto issue = [&](int g, int b) {
      const bool live = g < s1;
      dma_x2(lds0 + b * kXStage + wid * 2048, buffer_rsrc(xt + g * 32, live ? xbytes - g * 64 : 0), xvo[0],
             xvo[1]);
      if (wid < 4) {
        dma_x1(lds0 + kOffC + b * kCStage + wid * 1024, buffer_rsrc(pt + g * 16, live ? cbytes - g * 16 : 0), cvo);
      } else {
        const bool sl = live && ((g & 7) == 0 || g == s0);
        dma_x1(sl ? lds0 + kOffS + ((g >> 3) & 1) * kSBlock + (wid - 4) * 1024 : lds0 + kOffJunk,
               buffer_rsrc(st + (g & ~7), sl ? sbytes - (g & ~7) * 2 : 0), svo);
      }
    };
    // the code words and scale of this lane's B fragment for group h (stage buffer b): column
    // 32 w + l % 32, word 2 kk + l / 32 (codes 16 kk + 8 (l / 32) .. + 7)
    struct Codes {
      uint32_t w[2];  // [kk]
      uint32_t s;     // fp16 bits
    };
    const int bn = 32 * wid + fr;  // this lane's column of the tile
    auto read_codes = [&](int h, int b, Codes& cd) {
      const uint32_t* cw = reinterpret_cast<const uint32_t*>(lds + kOffC + b * kCStage + bn * 16);
      cd.w[0] = cw[fh];
      cd.w[1] = cw[2 + fh];
      cd.s = *reinterpret_cast<const uint16_t*>(lds + kOffS + ((h >> 3) & 1) * kSBlock + bn * 16 + (h & 7) * 2);
    };
    // bf16 B fragment of step kk: per 8 codes, the even and odd nibbles as bytes in offset
    // binary (q + 8), each converted to float, and s * (q + 8) - 8 s in one fma (exact: it
    // equals s * q, which fp32 holds), rounded to bf16 in pairs
    struct BFrag {
      bf16x8 v[kSplit ? 2 : 1];  // [0]: s * q (or s_hi * q), [1]: s_lo * q
    };
    auto make_b = [&](const Codes& cd, int kk, BFrag& bf) {
      const float sc = f16_bits_to_f32(static_cast<uint16_t>(cd.s));
      const uint32_t word = cd.w[kk];
      const uint32_t ev = (word & 0x0F0F0F0Fu) ^ 0x08080808u;
      const uint32_t od = ((word >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
      float qe[4], qo[4];  // q + 8 of the even and odd nibbles
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        qe[p] = static_cast<float>((ev >> (8 * p)) & 0xFFu);
        qo[p] = static_cast<float>((od >> (8 * p)) & 0xFFu);
      }
      auto part = [&](float s, bf16x8& out) {  // bf16 of s * q (exact when s * q fits bf16)
        const float ms = -8.0f * s;
        uint32_t h[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float w0 = __builtin_fmaf(s, qe[p], ms);
          const float w1 = __builtin_fmaf(s, qo[p], ms);
          h[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{w0, w1}, bf16x2));
        }
        out = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
      };
      if constexpr (kSplit) {
        // s rounded to 5 significant bits (fraction bits below the top 4 cleared, half rounded up)
        const float s_hi = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, sc) + 0x00040000u) & 0xFFF80000u);
        part(s_hi, bf.v[0]);
        part(sc - s_hi, bf.v[1]);
      } else {
        part(sc, bf.v[0]);
      }
    };

    f32x16 acc[8];
    // A fragments of one 16-code step (all 256 x rows)
    auto load_a = [&](int b, int kk, bf16x8 (&af)[8]) {
      const uint8_t* xb = lds + b * kXStage;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 32 * i + fr;
        af[i] = *reinterpret_cast<const bf16x8*>(xb + r * 64 + gswz(r, 2 * kk + fh));
      }
    };
    // the products of one step; `first` starts the sums from zero
    auto mma = [&](const bf16x8 (&af)[8], const BFrag& bf, auto first) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (decltype(first)::value)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf.v[0], zero16, 0, 0, 0);
        else
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf.v[0], acc[i], 0, 0, 0);
        if constexpr (kSplit) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf.v[1], acc[i], 0, 0, 0);
      }
    };
    // each product followed by one LDS read of the next step and kV vector instructions of the
    // next step's B fragment
    auto pattern = [&](auto kv) {
      constexpr int V = decltype(kv)::value;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, kSplit ? 2 : 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);               // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, kSplit ? V + 2 : V, 0);  // VALU
      }
    };
    // stage synchronisation: this wave's loads up to two stages back have landed and its LDS
    // reads are done; after the barrier those loads are visible to all wavefronts and nobody
    // reads the stage buffer that the next loads overwrite
    auto stage_sync = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * kOpsPerStage));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };

    // Group g: x and codes in stage buffer g % GNB.  Stage g starts with one barrier: before
    // it this wave's loads up to g + 1 have landed (those of g + 2 and g + 3 stay in flight)
    // and its LDS reads are done; after it the loads of g + 4 go to the buffer of g - 1, which
    // nobody reads any more.  Step 0 multiplies the fragments of kk = 0 of g (set X, prepared
    // during stage g - 1) while those of kk = 1 (set Y) are prepared and the codes of g + 1 are
    // read; step 1 multiplies set Y while set X is refilled with kk = 0 of g + 1.
    bf16x8 ax[8], ay[8];
    BFrag bx, by;
    Codes cg, cn;
    int gb = s0 % GNB;  // stage buffer of group g
    issue(s0, gb);
    issue(s0 + 1, sbuf(gb, 1));
    issue(s0 + 2, sbuf(gb, 2));
    issue(s0 + 3, sbuf(gb, 3));
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * kOpsPerStage));  // own loads of s0
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    read_codes(s0, gb, cg);
    load_a(gb, 0, ax);
    make_b(cg, 0, bx);
    for (int g = s0; g < s1; ++g) {
      stage_sync();
      issue(g + 4, sbuf(gb, 4));
      read_codes(g + 1, sbuf(gb, 1), cn);  // (past the range: empty codes, never used)
      load_a(gb, 1, ay);
      make_b(cg, 1, by);
      if (g == s0)
        mma(ax, bx, std::true_type{});
      else
        mma(ax, bx, std::false_type{});
      pattern(std::integral_constant<int, 3>{});
      load_a(sbuf(gb, 1), 0, ax);  // (past the range: a stale buffer, never used)
      make_b(cn, 0, bx);
      mma(ay, by, std::false_type{});
      pattern(std::integral_constant<int, 3>{});
      cg = cn;
      gb = sbuf(gb, 1);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    if (s0 == 0 && s1 == G) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        gstore_block(y, y_dtype, M, N, m0 + 32 * i, n0 + 32 * wid, acc[i], lane);
        asm volatile("" ::: "memory");
      }
    } else {
      float* slot = ws + (int64_t)(2 * lb + (it == it_begin ? 0 : 1)) * kGTileElems;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          *reinterpret_cast<f32x4*>(slot + gpart_off(wid, i, a, lane)) =
              f32x4{acc[i][4 * a], acc[i][4 * a + 1], acc[i][4 * a + 2], acc[i][4 * a + 3]};
          asm volatile("" ::: "memory");
        }
    }
    it += s1 - s0;
  }
}

// Tiles whose groups were spread over several workgroups: sum the partial tiles in the order of
// their K ranges, then store.  One workgroup of 8 wavefronts per (tile, block row i); wavefront
// w sums its own block (rows 32 i.., columns 32 w..).
__global__ __launch_bounds__(kGThreads) void gemm_fixup_kernel(void* __restrict__ y, int y_dtype, int M, int N,
                                                               int G, int tn_count, int chunk,
                                                               const float* __restrict__ ws) {
  const int t = blockIdx.x >> 3;
  const int i = blockIdx.x & 7;
  const int first = static_cast<int>((int64_t)t * G / chunk);
  const int last = static_cast<int>(((int64_t)t * G + G - 1) / chunk);
  if (first == last) return;
  const int tm = t / tn_count, tn = t - tm * tn_count;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  f32x16 v;
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = 0.0f;
  for (int b = first; b <= last; ++b) {
    const int slot = 2 * b + ((int64_t)b * chunk >= (int64_t)t * G ? 0 : 1);
    const float* p = ws + (int64_t)slot * kGTileElems;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(p + gpart_off(wid, i, a, lane));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * a + e] += q[e];
    }
  }
  gstore_block(y, y_dtype, M, N, tm * GT + 32 * i, tn * GT + 32 * wid, v, lane);
}

// Schedule of one pass of the tiled kernel: stream-K ranges of `chunk` (tile, K-group)
// iterations, one per workgroup, and the scratch their partial tiles need (two fp32 tiles per
// workgroup, only when some tile is split over workgroups).
struct DqPlan {
  int64_t tn_count, tiles, G, total, chunk, nblk, per_xcd;
  bool partial;
  size_t ws_need;
};

constexpr size_t kGSlotPair = size_t(2) * kGTileElems * sizeof(float);

void dq_finish(DqPlan& p) {
  p.nblk = (p.total + p.chunk - 1) / p.chunk;
  p.partial = p.nblk > 1 && p.chunk % p.G != 0;
  p.ws_need = p.partial ? size_t(p.nblk) * kGSlotPair : 0;
  p.per_xcd = (p.nblk + 7) / 8;
}

// The fastest schedule (SIZE_MAX) or the fastest whose scratch fits ws_bytes: the most
// workgroups whose partial tiles fit, or one whole tile per workgroup (no scratch), whichever
// runs more workgroups.
DqPlan plan_dq(int64_t m, int64_t N, int64_t K, size_t ws_bytes) {
  DqPlan p;
  p.G = K / 32;
  const int64_t tm_count = (m + GT - 1) / GT;
  p.tn_count = (N + GT - 1) / GT;
  p.tiles = tm_count * p.tn_count;
  p.total = p.tiles * p.G;
  int64_t nblk = (p.total + kGMinChunk - 1) / kGMinChunk;
  if (nblk > kGMaxBlocks) nblk = kGMaxBlocks;
  p.chunk = (p.total + nblk - 1) / nblk;
  dq_finish(p);
  if (p.ws_need <= ws_bytes) return p;
  const int64_t fit = static_cast<int64_t>(ws_bytes / kGSlotPair);
  DqPlan q = p;
  q.chunk = q.G;
  dq_finish(q);
  if (fit >= 2) {
    DqPlan r = p;
    r.chunk = (r.total + fit - 1) / fit;
    dq_finish(r);
    if (r.ws_need <= ws_bytes && r.nblk > q.nblk) return r;
  }
  return q;
}

int launch_dq_pass(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16, int64_t N,
                    int64_t K, void* y, int y_dtype, bool exact, void* ws_ptr, size_t ws_bytes, hipStream_t s) {
  const DqPlan p = plan_dq(m, N, K, ws_ptr != nullptr ? ws_bytes : 0);
  if (p.total > 0x3FFFFFFF) return W4Q_EUNSUPPORTED;
  float* ws = p.partial ? static_cast<float*>(ws_ptr) : nullptr;
  const dim3 grid(static_cast<unsigned>(8 * p.per_xcd));
  if (exact)
    hipLaunchKernelGGL(gemm_dq_kernel<true>, grid, dim3(kGThreads), 0, s, x, static_cast<int>(m), packed, s16,
                       static_cast<int>(N), static_cast<int>(K), y, y_dtype, static_cast<int>(p.tn_count),
                       static_cast<int>(p.total), static_cast<int>(p.chunk), static_cast<int>(p.nblk),
                       static_cast<int>(p.per_xcd), ws);
  else
    hipLaunchKernelGGL(gemm_dq_kernel<false>, grid, dim3(kGThreads), 0, s, x, static_cast<int>(m), packed, s16,
                       static_cast<int>(N), static_cast<int>(K), y, y_dtype, static_cast<int>(p.tn_count),
                       static_cast<int>(p.total), static_cast<int>(p.chunk), static_cast<int>(p.nblk),
                       static_cast<int>(p.per_xcd), ws);
  int rc = w4q_launch_status();
  if (p.partial && rc == W4Q_OK) {
    hipLaunchKernelGGL(gemm_fixup_kernel, dim3(static_cast<unsigned>(8 * p.tiles)), dim3(kGThreads), 0, s, y,
                       y_dtype, static_cast<int>(m), static_cast<int>(N), static_cast<int>(p.G),
                       static_cast<int>(p.tn_count), static_cast<int>(p.chunk), ws);
    rc = w4q_launch_status();
  }
  return rc;
}

}  // namespace
}  // namespace w4q

using namespace w4q;

// output tiles of the per-group kernel: 256-row tiles (8 wavefronts share one expansion of the
// codes) when they still give at least one tile per compute unit, 128-row tiles otherwise
static int64_t group_tiles(int64_t m, int64_t d_out, bool* big) {
  const int64_t gn = (d_out + BN - 1) / BN;
  const int64_t gm4 = (m + 255) / 256, gm2 = (m + 127) / 128;
  *big = gm4 * gn >= 256;
  return (*big ? gm4 : gm2) * gn;
}

// exact weights, any shape: one K-group per step, scale applied per group on the vector ALUs
static int launch_group(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                 int64_t d_out, int64_t d_in, void* y, int y_dtype, hipStream_t s) {
  if (d_in / kGroup > 0x7FFFFFFF) return W4Q_EUNSUPPORTED;
  const int64_t gn = (d_out + BN - 1) / BN;
  bool big;
  const int64_t tiles = group_tiles(m, d_out, &big);
  const int64_t per_xcd = (tiles + 7) / 8;
  if (8 * per_xcd > 0x7FFFFFFF) return W4Q_EUNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(8 * per_xcd));
  if (big)
    hipLaunchKernelGGL(gemm_group_kernel<4>, grid, dim3(64 * 4 * WN), 0, s, x, m, packed, s16, d_out, d_in, y,
                       y_dtype, gn, tiles, per_xcd);
  else
    hipLaunchKernelGGL(gemm_group_kernel<2>, grid, dim3(64 * 2 * WN), 0, s, x, m, packed, s16, d_out, d_in, y,
                       y_dtype, gn, tiles, per_xcd);
  return w4q_launch_status();
}

// the tiled kernel needs 16-byte scale rows (d_in % 256 == 0) and 32-bit buffer offsets into
// the codes and scales; x is taken in passes of whole 256-row tiles that fit them too
static bool tiled_ok(int64_t d_out, int64_t d_in) {
  return d_in % 256 == 0 && d_out * (d_in / 2) < 0x7FFFFFFF && 256 * d_in * 2 < 0x7FFFFFFF;
}
static int64_t pass_rows(int64_t d_in) { return (0x7FFFFFFF / (2 * d_in)) / GT * GT; }

// exact weights go to the split-scale tiled kernel only while the per-group kernel would leave
// compute units idle (fewer than 256 output tiles) and the tiled kernel can take the shape
static bool exact_on_tiled(int64_t m, int64_t d_out, int64_t d_in) {
  bool big;
  return tiled_ok(d_out, d_in) && group_tiles(m, d_out, &big) < 256;
}

size_t w4q_gemm_workspace(int64_t m, int64_t d_out, int64_t d_in, int w_mode) {
  if (w_mode == 0 && (m <= 16 || !exact_on_tiled(m, d_out, d_in))) return 0;
  if (!tiled_ok(d_out, d_in)) return 0;
  const int64_t rows = pass_rows(d_in);
  const int64_t first = m < rows ? m : rows;
  const int64_t last = m % rows == 0 ? first : m % rows;
  const size_t a = plan_dq(first, d_out, d_in, SIZE_MAX).ws_need;
  const size_t b = plan_dq(last, d_out, d_in, SIZE_MAX).ws_need;
  return a > b ? a : b;
}

int w4q_launch_gemm(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                    int64_t d_out, int64_t d_in, void* y, int y_dtype, int w_mode, void* ws,
                    size_t ws_bytes, hipStream_t s) {
  if (w_mode == 0) {
    // exact weights: the per-group kernel while it has a tile for every compute unit; below
    // that, the stream-K tiled kernel with split weights (twice the matrix-core work, but the
    // K dimension spread over all compute units) when the caller's scratch holds its partial
    // tiles
    if (!exact_on_tiled(m, d_out, d_in) || ws == nullptr || ws_bytes < w4q_gemm_workspace(m, d_out, d_in, 0))
      return launch_group(x, m, packed, s16, d_out, d_in, y, y_dtype, s);
  }
  if (!tiled_ok(d_out, d_in)) return W4Q_EUNSUPPORTED;
  const int64_t rows = pass_rows(d_in);
  const int64_t ob = y_dtype == 0 ? 4 : 2;
  for (int64_t r0 = 0; r0 < m; r0 += rows) {
    const int64_t mr = m - r0 < rows ? m - r0 : rows;
    const int rc = launch_dq_pass(x + r0 * d_in, mr, packed, s16, d_out, d_in,
                                  static_cast<uint8_t*>(y) + r0 * d_out * ob, y_dtype, w_mode == 0, ws,
                                  ws_bytes, s);
    if (rc != W4Q_OK) return rc;
  }
  return W4Q_OK;
}

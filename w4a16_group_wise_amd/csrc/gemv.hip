// gemv.hip -- W4A16 product for 1..16 activation rows (decode): streams the packed INT4 codes
// and fp16 scales from HBM once.  One row runs on the vector ALUs (below, and the persistent
// stream kernel further down); 2..16 rows run on the matrix cores (the section "2..16
// activation rows").
//
// Method: model card "Opt.Gear-1B-qat-int4-per-channel-unquantized" (W4A16: INT4 weights with
// 16-bit activations; weight memory and bandwidth set the speed) with the group-32 symmetric
// grid of blog "Opt.Gear-QAT: Preserving On-Device Performance with QAT".
//   y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] * q[n][k]
//
// Vector mapping: a group of 32 codes is one 16-byte load, so a lane owns one group column; LPR lanes
// (a power of two dividing G) cover one row per chunk of LPR groups, and a wavefront works on
// 64 / LPR rows at once, RS row-steps deep, walking the chunks along d_in.  Loads of a row are
// contiguous (LPR * 16 bytes).  The lane keeps its group's activations as bf16 pairs in
// registers, reused for all the rows of the wavefront.
//
// Codes: every product x * q is formed exactly from the unbiased code.  A dword of 8
// two's-complement nibbles is spread into two dwords of signed bytes, each nibble in the high
// half of its byte (one shift and two masks), so that every byte holds 16 q; one conversion per
// byte (byte select with sign extension) gives 16 q in fp32.  The vector kernels accumulate
// x * 16q with fused multiply-adds; the matrix-core kernel packs 16 q as bf16 (small integers,
// exact) for the products.  The group's scale, times 1/16 (exact for every fp16 scale),
// multiplies the group's sum, in fp32.  So the rounding error of a product is a few 2^-24 of
// sum |x * w_hat|, whatever the codes and the spread of x (an offset encoding of the codes,
// x * (q + c) - x * c, would carry an error of order 2^-24 c sum |x|, far above the product when
// the codes are mostly zero where |x| is large).  Launches of at least 48 MB of codes take the
// exact bf16 code pairs from a table in LDS instead (see the stream kernel).  The next chunk's
// codes, scales and activations are loaded while the current chunk is being reduced.
#include <atomic>

#include "common.hpp"

namespace w4q {
namespace {

constexpr int kThreads = 256;

// the 8 codes of a dword of two's-complement nibbles (nibble i at bits 4i..4i+3), times 16, in
// order: nibble i goes to the high half of byte i / 2 of one of two dwords, whose signed bytes
// convert exactly (one byte-select conversion each)
__device__ __forceinline__ void codes16_f32(uint32_t v, float* c) {
  const uint32_t ev = (v << 4) & 0xF0F0F0F0u;  // nibbles 0, 2, 4, 6
  const uint32_t od = v & 0xF0F0F0F0u;         // nibbles 1, 3, 5, 7
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[2 * j] = static_cast<float>(static_cast<int8_t>(ev >> (8 * j)));
    c[2 * j + 1] = static_cast<float>(static_cast<int8_t>(od >> (8 * j)));
  }
}

// the same 8 values (16 q) as four bf16 pairs (codes 2j, 2j + 1), exact
__device__ __forceinline__ u32x4 codes16_bf16x8(uint32_t v) {
  float c[8];
  codes16_f32(v, c);
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    p[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{c[2 * j], c[2 * j + 1]}, bf16x2));
  return u32x4{p[0], p[1], p[2], p[3]};
}

// a group's fp16 scale times 1/16, the factor the codes above carry
__device__ __forceinline__ float scale16(uint32_t bits) {
  return f16_bits_to_f32(static_cast<uint16_t>(bits)) * 0.0625f;
}

// 8 activations (4 dwords of bf16 pairs) as fp32, in order
__device__ __forceinline__ void x_f32(const u32x4 d, float* o) {
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[2 * j] = bf16_lo(w[j]);
    o[2 * j + 1] = bf16_hi(w[j]);
  }
}

// sum_{i < 8} x[i] * 16 * code i of v, added to a (fused multiply-adds, exact products)
__device__ __forceinline__ float dot8(const float* x, uint32_t v, float a) {
  float c[8];
  codes16_f32(v, c);
#pragma unroll
  for (int i = 0; i < 8; ++i) a = __builtin_fmaf(x[i], c[i], a);
  return a;
}

template <int MT, int RS>
struct Chunk {
  u32x4 code[RS];
  uint32_t sc[RS];
  u32x4 xv[MT][4];
};

// The product for the rows of workgroup `block` (of a grid covering d_out).
template <int MT, int LPR, int RS>
__device__ __forceinline__ void gemv_body(const uint16_t* __restrict__ x, int m_rows,
                                          const uint8_t* __restrict__ packed,
                                          const uint16_t* __restrict__ s16, int64_t d_out, int64_t d_in,
                                          void* __restrict__ y, int y_dtype, int64_t block) {
  constexpr int RPS = 64 / LPR;  // rows per row-step
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;
  const int j = lane % LPR;
  const int64_t wave = block * (kThreads / 64) + threadIdx.x / 64;
  const int64_t row0 = wave * (RPS * RS);
  if (row0 >= d_out) return;  // uniform per wavefront
  const int G = static_cast<int>(d_in / kGroup);
  const int nchunk = G / LPR;

  // per row-step base pointers (64-bit once), then 32-bit offsets per chunk
  const uint8_t* prow[RS];
  const uint16_t* srow[RS];
  bool rok[RS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const int64_t n = row0 + rs * RPS + sub;
    rok[rs] = n < d_out;
    const int64_t nn = rok[rs] ? n : 0;
    prow[rs] = packed + nn * (d_in / 2) + j * 16;
    srow[rs] = s16 + nn * G + j;
  }
  const uint16_t* xrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xrow[m] = x + (m < m_rows ? m : 0) * d_in + j * kGroup;

  auto load = [&](int c, Chunk<MT, RS>& k) {
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      k.code[rs] = *reinterpret_cast<const u32x4*>(prow[rs] + c * (LPR * 16));
      k.sc[rs] = srow[rs][c * LPR];
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int b = 0; b < 4; ++b) k.xv[m][b] = *reinterpret_cast<const u32x4*>(xrow[m] + c * (LPR * kGroup) + 8 * b);
  };

  float acc[RS][MT];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[rs][m] = 0.0f;

  auto compute = [&](const Chunk<MT, RS>& cur) {
    float sums[RS][MT];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs)
#pragma unroll
      for (int m = 0; m < MT; ++m) sums[rs][m] = 0.0f;
    // 8 activations at a time (as fp32), against dword b of every row's codes
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float xf[8];
        x_f32(m < m_rows ? cur.xv[m][b] : u32x4{0u, 0u, 0u, 0u}, xf);
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) sums[rs][m] = dot8(xf, cur.code[rs][b], sums[rs][m]);
      }
    }
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      const float sc = scale16(cur.sc[rs]);
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[rs][m] = __builtin_fmaf(sc, sums[rs][m], acc[rs][m]);
    }
  };

  // two register sets: the loads of one chunk are in flight while the other is reduced
  // (the empty asm with a memory clobber keeps each batch of loads where it is issued)
  Chunk<MT, RS> ca, cb;
  load(0, ca);
  int c = 0;
  for (; c + 1 < nchunk; c += 2) {
    load(c + 1, cb);
    asm volatile("" ::: "memory");
    compute(ca);
    if (c + 2 < nchunk) load(c + 2, ca);
    asm volatile("" ::: "memory");
    compute(cb);
  }
  if (c < nchunk) compute(ca);
  // reduce the LPR lane partials of each row (fixed butterfly order)
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const int64_t n = row0 + rs * RPS + sub;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[rs][m];
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      if (j == 0 && rok[rs] && m < m_rows) {
        if (y_dtype == 0)
          reinterpret_cast<float*>(y)[m * d_out + n] = v;
        else
          reinterpret_cast<uint16_t*>(y)[m * d_out + n] = f32_to_bf16_bits(v);
      }
    }
  }
}

template <int MT, int LPR, int RS>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint16_t* __restrict__ x, int m_rows,
                                                        const uint8_t* __restrict__ packed,
                                                        const uint16_t* __restrict__ s16,
                                                        int64_t d_out, int64_t d_in,
                                                        void* __restrict__ y, int y_dtype) {
  gemv_body<MT, LPR, RS>(x, m_rows, packed, s16, d_out, d_in, y, y_dtype, blockIdx.x);
}

// ---- 2..16 activation rows on the matrix cores ------------------------------------------
//
// One v_mfma_f32_16x16x32_bf16 per (group, 16 rows of W) forms the 16 x 16 block of per-group
// sums sum_{k in g} x[m][k] * q[n][k] for all activation rows at once (rows past m_rows repeat
// the last one and are never stored), from the codes as exact bf16 integers; the group's scale
// is applied in fp32.  A operand: lane (q, m) = (lane / 16, lane % 16) holds x[m][32 g + 8 q + e]
// (e = 0..7); B operand: lane (q, n) holds the 8 codes of W row n at the same offsets.  The
// result: lane (q, n) holds rows m = 4 q + r of column n.
//
// A workgroup owns 32 rows of W (two tiles; 16 rows, one tile, when d_out < 8192, where two
// would leave too few workgroups); its wavefronts take d_in's 8-group batches
// round-robin.  Each wavefront keeps two batches of codes and scales in flight: those of its next
// batch are issued before the current one is reduced; the activations (L2-resident) are loaded
// one batch ahead, right after the previous batch's products.  Codes: lane (q, n) loads the whole group 4 h + q of row n
// (16 rows x 64 contiguous bytes per instruction), and a 4 x 4 transpose across the lanes q
// gives every lane dword q of each of the four groups.  Scales: one 16-byte load of the batch's
// 8 scales per row when G % 8 == 0 (then every batch start is 16-byte aligned), else one
// 2-byte load per group.  The wavefronts' partial results are added in LDS in a fixed order.
constexpr int kMmaWaves = 8;
constexpr int kMmaBatch = 8;

// 4 x 4 transpose across the 16-lane rows R = lane / 16: on entry v[j] of row R holds element
// (R, j), on exit element (j, R).  The 32-lane swap exchanges the off-diagonal 2 x 2 blocks,
// the 16-lane swap the off-diagonal elements inside each block.
__device__ __forceinline__ void transpose4(u32x4& v) {
  uint32_t a0 = v.x, a1 = v.y, a2 = v.z, a3 = v.w;
  auto s32 = [](uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    a = r0;
    b = r1;
  };
  auto s16 = [](uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    a = r0;
    b = r1;
  };
  s32(a0, a2);
  s32(a1, a3);
  s16(a0, a1);
  s16(a2, a3);
  v = u32x4{a0, a1, a2, a3};
}

template <int kMmaTiles>
struct MmaBatch {
  u32x4 cv[kMmaBatch / 4][kMmaTiles];  // codes (transposed after arrival)
  u32x4 sc[kMmaTiles];                 // 8 scales per row (vector path)
  uint32_t s1[kMmaBatch][kMmaTiles];   // one scale per group (2-byte path)
};

// kMmaTiles: 16-row tiles of W per workgroup (1 or 2); kWaves: wavefronts per workgroup (8, or
// 16 for long rows, where each still gets two batches or more)
template <bool kVecScales, int kMmaTiles, int kWaves = kMmaWaves>
__global__ __launch_bounds__(kWaves * 64) void gemv_mma_kernel(const uint16_t* __restrict__ x, int m_rows,
                                                                  const uint8_t* __restrict__ packed,
                                                                  const uint16_t* __restrict__ s16,
                                                                  int64_t d_out, int64_t d_in,
                                                                  void* __restrict__ y, int y_dtype) {
  __shared__ float part[kWaves][kMmaTiles][4][64];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4, nl = lane & 15;
  const int G = static_cast<int>(d_in / kGroup);
  const int nbat = (G + kMmaBatch - 1) / kMmaBatch;
  const int64_t nbase = (int64_t)blockIdx.x * (16 * kMmaTiles);

  // rows of W past d_out read the last row (their columns are never stored)
  const uint8_t* prow[kMmaTiles];
  const uint16_t* srow[kMmaTiles];
#pragma unroll
  for (int t = 0; t < kMmaTiles; ++t) {
    const int64_t n = nbase + 16 * t + nl;
    const int64_t nn = n < d_out ? n : d_out - 1;
    prow[t] = packed + nn * (d_in / 2);
    srow[t] = s16 + nn * G;
  }
  const int mr = nl < m_rows ? nl : m_rows - 1;
  const uint16_t* xrow = x + (int64_t)mr * d_in + 8 * q;
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  // the loads of batch b, all issued at once; groups past G repeat the last one.  Every loaded
  // value passes through an empty asm, so no load can sink into the product of its group.
  auto load = [&](int b, MmaBatch<kMmaTiles>& B) {
    const int gb = b * kMmaBatch;
#pragma unroll
    for (int h = 0; h < kMmaBatch / 4; ++h) {
      const int g = gb + 4 * h + q < G ? gb + 4 * h + q : G - 1;
#pragma unroll
      for (int t = 0; t < kMmaTiles; ++t) B.cv[h][t] = *reinterpret_cast<const u32x4*>(prow[t] + (int64_t)g * 16);
    }
    if constexpr (kVecScales) {
#pragma unroll
      for (int t = 0; t < kMmaTiles; ++t) B.sc[t] = *reinterpret_cast<const u32x4*>(srow[t] + gb);
    } else {
#pragma unroll
      for (int i = 0; i < kMmaBatch; ++i) {
        const int g = gb + i < G ? gb + i : G - 1;
#pragma unroll
        for (int t = 0; t < kMmaTiles; ++t) B.s1[i][t] = srow[t][g];
      }
    }
#pragma unroll
    for (int h = 0; h < kMmaBatch / 4; ++h)
#pragma unroll
      for (int t = 0; t < kMmaTiles; ++t) asm volatile("" : "+v"(B.cv[h][t]));
    if constexpr (kVecScales) {
#pragma unroll
      for (int t = 0; t < kMmaTiles; ++t) asm volatile("" : "+v"(B.sc[t]));
    } else {
#pragma unroll
      for (int i = 0; i < kMmaBatch; ++i)
#pragma unroll
        for (int t = 0; t < kMmaTiles; ++t) asm volatile("" : "+v"(B.s1[i][t]));
    }
  };
  // the activations of batch b (from L2: issued after the previous batch's products, they land
  // while the codes, loaded a batch earlier, are still arriving)
  u32x4 xv[kMmaBatch];
  auto load_x = [&](int b) {
    const int gb = b * kMmaBatch;
#pragma unroll
    for (int i = 0; i < kMmaBatch; ++i) {
      const int g = gb + i < G ? gb + i : G - 1;
      xv[i] = *reinterpret_cast<const u32x4*>(xrow + (int64_t)g * kGroup);
    }
#pragma unroll
    for (int i = 0; i < kMmaBatch; ++i) asm volatile("" : "+v"(xv[i]));
  };

  f32x4 acc[kMmaTiles];
#pragma unroll
  for (int t = 0; t < kMmaTiles; ++t) acc[t] = zero4;

  auto compute = [&](int b, MmaBatch<kMmaTiles>& B) {
    const int nb = G - b * kMmaBatch < kMmaBatch ? G - b * kMmaBatch : kMmaBatch;
#pragma unroll
    for (int h = 0; h < kMmaBatch / 4; ++h)
#pragma unroll
      for (int t = 0; t < kMmaTiles; ++t) transpose4(B.cv[h][t]);
#pragma unroll
    for (int i = 0; i < kMmaBatch; ++i) {
      if (i >= nb) break;  // wavefront-uniform
      const bf16x8 a = __builtin_bit_cast(bf16x8, xv[i]);
#pragma unroll
      for (int t = 0; t < kMmaTiles; ++t) {
        const f32x4 dv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a, __builtin_bit_cast(bf16x8, codes16_bf16x8(B.cv[i / 4][t][i % 4])), zero4, 0, 0, 0);
        uint32_t sbits;
        if constexpr (kVecScales)
          sbits = B.sc[t][i / 2] >> (16 * (i % 2));
        else
          sbits = B.s1[i][t];
        const float sc = scale16(sbits);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = __builtin_fmaf(sc, dv[r], acc[t][r]);
      }
    }
  };

  // the wavefronts take the batches round-robin (wavefront w: w, w + S, ... for S wavefronts), so at any time a
  // workgroup reads a few hundred contiguous bytes of each of its rows; two register sets: the
  // next batch is in flight while the current one is reduced
  constexpr int S = kWaves;
  MmaBatch<kMmaTiles> B0, B1;
  if (wid < nbat) {
    load(wid, B0);
    load_x(wid);
  }
  for (int b = wid; b < nbat; b += 2 * S) {
    if (b + S < nbat) load(b + S, B1);
    compute(b, B0);
    if (b + S >= nbat) break;
    load_x(b + S);
    if (b + 2 * S < nbat) load(b + 2 * S, B0);
    compute(b + S, B1);
    if (b + 2 * S < nbat) load_x(b + 2 * S);
  }

#pragma unroll
  for (int t = 0; t < kMmaTiles; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wid][t][r][lane] = acc[t][r];
  __syncthreads();
  // outputs: tile t, activation row m, column c; wavefront partials in order
  for (int o = threadIdx.x; o < kMmaTiles * 256; o += kWaves * 64) {
    const int t = o >> 8, m = (o >> 4) & 15, c = o & 15;
    const int src = 16 * (m >> 2) + c;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += part[w][t][m & 3][src];
    const int64_t n = nbase + 16 * t + c;
    if (m < m_rows && n < d_out) {
      if (y_dtype == 0)
        reinterpret_cast<float*>(y)[m * d_out + n] = v;
      else
        reinterpret_cast<uint16_t*>(y)[m * d_out + n] = f32_to_bf16_bits(v);
    }
  }
}

// ---- one activation row: a persistent stream over many problems --------------------------
//
// The rows of every problem are cut into items of RPS * RS rows (one wavefront's row-steps).
// Each wavefront of a fixed, fully resident grid takes the items w, w + W, w + 2W, ... (W = all
// wavefronts of the grid) and walks them as one stream of (item, chunk) units: the loads of the
// next unit -- which may belong to the next item or the next problem -- are in flight while the
// current unit is reduced, so the stream does not drain at item boundaries.  When the last chunk
// of an item is reduced, its rows are finished (lane reduction, store) and the accumulators
// restart.  Problems are numbered in the order given; first[p] is the first item of problem p.
constexpr int kMaxGroup = 64;
struct GroupArgs {
  const uint16_t* x[kMaxGroup];
  const uint8_t* packed[kMaxGroup];
  const uint16_t* s16[kMaxGroup];
  void* y[kMaxGroup];
  int d_out[kMaxGroup];
  int d_in[kMaxGroup];
  int first[kMaxGroup + 1];
  int n;
  int y_dtype;
};

__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(v))));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(v >> 32))));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// global (not generic) address space: loads through these are global_load with an SGPR base
#define W4Q_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ W4Q_GLOBAL T* global_ptr(T* p) {
  return (W4Q_GLOBAL T*)(p);
}

template <int RS>
struct Src {  // where the loads of one item come from: wave-uniform bases, per-lane 32-bit offsets
  const W4Q_GLOBAL uint8_t* pbase[RS];   // codes of each row (one row per row-step) or of the first
  const W4Q_GLOBAL uint16_t* sbase[RS];  // scales likewise
  const W4Q_GLOBAL uint16_t* xbase;      // activations
  uint32_t poff[RS];                     // byte offset of (row, lane column) from pbase
  uint32_t soff[RS];                     // element offset of (row, lane group) from sbase
  int nchunk;
};

__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_uint(float f) { return __builtin_bit_cast(uint32_t, f); }
// lanes 32..63 of a trade places with lanes 0..31 of b
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(as_uint(a), as_uint(b), false, false);
  const uint32_t u0 = r[0], u1 = r[1];
  a = as_float(u0);
  b = as_float(u1);
}
// 16-lane rows 1 and 3 of a trade places with rows 0 and 2 of b
__device__ __forceinline__ void swap_rows(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(as_uint(a), as_uint(b), false, false);
  const uint32_t u0 = r[0], u1 = r[1];
  a = as_float(u0);
  b = as_float(u1);
}
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, false));
}

// code byte e (codes 2j and 2j + 1 in its low and high nibble) -> the exact bf16 pair of the two
// codes (small integers), low half = code 2j
__device__ __forceinline__ uint32_t lut_pair(int e) {
  const int lo = static_cast<int>(static_cast<uint32_t>(e) << 28) >> 28;  // sign-extended low nibble
  const int hi = static_cast<int>(static_cast<uint32_t>(e) << 24) >> 28;  // sign-extended high nibble
  const uint32_t blo = __builtin_bit_cast(uint32_t, static_cast<float>(lo)) >> 16;  // exact in bf16
  const uint32_t bhi = __builtin_bit_cast(uint32_t, static_cast<float>(hi)) >> 16;
  return blo | (bhi << 16);
}

// threads per workgroup of the stream kernel: 512 with the code table (two workgroups of 64 KB of
// table per compute unit), 256 without
template <bool kLut>
constexpr int stream_threads() { return kLut ? 512 : 256; }

// The argument table is read where it is passed (the kernel arguments): the problem of an item
// is one ballot over first[] (the number of problems q >= 1 with first[q] <= item), then scalar
// reads of that problem's entries.  (Staging the table through LDS first put a barrier and an LDS
// round trip before the first code load: per-phase decode pass of the 36-layer stack 1262 ->
// 1205 us without it.)
template <int LPR, int RS, bool kLut>
__global__ __launch_bounds__(stream_threads<kLut>()) void gemv_stream_kernel(const GroupArgs t) {
  constexpr int kStreamThreads = stream_threads<kLut>();
  __shared__ uint32_t lut[kLut ? 256 * 64 : 1];
  constexpr int RPS = 64 / LPR;
  constexpr int ROWS = RPS * RS;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;
  const int j = lane % LPR;
  const int n = uniform_int(t.n);
  const int64_t nitems = uniform_int(t.first[n]);
  const int ydt = uniform_int(t.y_dtype);
  const int fq = lane >= 1 && lane < n ? t.first[lane] : 0x7FFFFFFF;
  const int64_t W = static_cast<int64_t>(uniform_int(static_cast<int>(gridDim.x))) * (kStreamThreads / 64);
  const int64_t w0 = static_cast<int64_t>(blockIdx.x) * (kStreamThreads / 64) + uniform_int(threadIdx.x / 64);
  const bool active = w0 < nitems;  // uniform per wavefront
  const uint32_t xoff = static_cast<uint32_t>(j * kGroup);
  const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;

  auto problem_of = [&](int64_t item) { return __builtin_popcountll(__ballot(fq <= item)); };
  auto setup = [&](int64_t item, Src<RS>& sr) {
    const int p = problem_of(item);
    const int64_t d_in = uniform_int(t.d_in[p]);
    const int64_t d_out = uniform_int(t.d_out[p]);
    const int G = static_cast<int>(d_in / kGroup);
    const int64_t r0 = (item - uniform_int(t.first[p])) * ROWS;
    const W4Q_GLOBAL uint8_t* pk = global_ptr(uniform_ptr(t.packed[p])) + r0 * (d_in / 2);
    const W4Q_GLOBAL uint16_t* sk = global_ptr(uniform_ptr(t.s16[p])) + r0 * G;
    sr.xbase = global_ptr(uniform_ptr(t.x[p]));
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      if constexpr (RPS == 1) {
        // one row per row-step: the row is wave-uniform, so it goes into the base
        const int64_t r = r0 + rs < d_out ? rs : 0;  // rows past the end read the first row; never stored
        sr.pbase[rs] = pk + r * (d_in / 2);
        sr.sbase[rs] = sk + r * G;
        sr.poff[rs] = static_cast<uint32_t>(j * 16);
        sr.soff[rs] = static_cast<uint32_t>(j);
      } else {
        const int lr = rs * RPS + sub;
        const uint32_t r = r0 + lr < d_out ? static_cast<uint32_t>(lr) : 0u;  // as above
        sr.pbase[rs] = pk;
        sr.sbase[rs] = sk;
        sr.poff[rs] = r * static_cast<uint32_t>(d_in / 2) + static_cast<uint32_t>(j * 16);
        sr.soff[rs] = r * static_cast<uint32_t>(G) + static_cast<uint32_t>(j);
      }
    }
    sr.nchunk = G / LPR;
  };
  auto load = [&](const Src<RS>& sr, int c, Chunk<1, RS>& k) {
    const W4Q_GLOBAL uint16_t* xb = sr.xbase + c * (LPR * kGroup);
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      const W4Q_GLOBAL uint8_t* pb = sr.pbase[rs] + c * (LPR * 16);
      const W4Q_GLOBAL uint16_t* sb = sr.sbase[rs] + c * LPR;
      // codes and scales are read once: non-temporal loads keep them from displacing cached data
      k.code[rs] = __builtin_nontemporal_load(
          reinterpret_cast<const W4Q_GLOBAL u32x4*>(pb + static_cast<uint64_t>(sr.poff[rs])));
      k.sc[rs] = __builtin_nontemporal_load(sb + static_cast<uint64_t>(sr.soff[rs]));
    }
#pragma unroll
    for (int b = 0; b < 4; ++b)
      k.xv[0][b] = *reinterpret_cast<const W4Q_GLOBAL u32x4*>(xb + static_cast<uint64_t>(xoff + 8 * b));
  };
  float acc[RS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) acc[rs] = 0.0f;
  // code byte k of word cw -> its two codes as an exact bf16 pair, from the lane's copy of the table
  // (dword e * 64 + lane: bank = lane, no conflict); the address is one byte permute
  auto pair = [&](uint32_t cw, int k) {
    const uint32_t addr = __builtin_amdgcn_perm(cw, lane4, 0x0C0C0400u | (static_cast<uint32_t>(4 + k) << 8));
    return __builtin_bit_cast(bf16x2, *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lut) + addr));
  };
  auto compute = [&](const Chunk<1, RS>& cur) {
    float sums[RS];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) sums[rs] = 0.0f;
    if constexpr (kLut) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t xw[4] = {cur.xv[0][b].x, cur.xv[0][b].y, cur.xv[0][b].z, cur.xv[0][b].w};
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) {
          const uint32_t cw = cur.code[rs][b];
#pragma unroll
          for (int k = 0; k < 4; ++k)  // activations 2k, 2k + 1 of dword b against codes 2k, 2k + 1
            sums[rs] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xw[k]), pair(cw, k), sums[rs], false);
        }
      }
#pragma unroll
      for (int rs = 0; rs < RS; ++rs)
        acc[rs] = __builtin_fmaf(f16_bits_to_f32(static_cast<uint16_t>(cur.sc[rs])), sums[rs], acc[rs]);
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float xf[8];
        x_f32(cur.xv[0][b], xf);
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) sums[rs] = dot8(xf, cur.code[rs][b], sums[rs]);
      }
#pragma unroll
      for (int rs = 0; rs < RS; ++rs)
        acc[rs] = __builtin_fmaf(scale16(cur.sc[rs]), sums[rs], acc[rs]);
    }
  };
  auto store = [&](void* y, int64_t row, float v) {
    if (ydt == 0)
      global_ptr(reinterpret_cast<float*>(y))[row] = v;
    else
      global_ptr(reinterpret_cast<uint16_t*>(y))[row] = f32_to_bf16_bits(v);
  };
  // reduce the lane partials of each row of `item` (fixed order), store, and restart the
  // accumulators
  auto finish = [&](int64_t item) {
    const int p = problem_of(item);
    const int64_t d_out = uniform_int(t.d_out[p]);
    void* y = uniform_ptr(t.y[p]);
    const int64_t r0 = (item - uniform_int(t.first[p])) * ROWS;
    if constexpr (LPR == 64 && RS == 4) {
      // four rows, 64 lanes each: halves and 16-lane rows trade places so that two rows are
      // summed per add; then 16-lane row k holds row k, reduced by rotations within the row
      float a0 = acc[0], a1 = acc[1], a2 = acc[2], a3 = acc[3];
      swap_halves(a0, a2);
      swap_halves(a1, a3);
      float s02 = a0 + a2;  // lanes 0..31: row 0, lanes 32..63: row 2
      float s13 = a1 + a3;  // lanes 0..31: row 1, lanes 32..63: row 3
      swap_rows(s02, s13);
      float v = s02 + s13;  // 16-lane row k: row k
      v += dpp<0x128>(v);   // row_ror:8
      v += dpp<0x124>(v);   // row_ror:4
      v += dpp<0x122>(v);   // row_ror:2
      v += dpp<0x121>(v);   // row_ror:1
      const int64_t row = r0 + (lane >> 4);
      if ((lane & 15) == 0 && row < d_out) store(y, row, v);
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) acc[rs] = 0.0f;
    } else {
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) {
        float v = acc[rs];
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        acc[rs] = 0.0f;
        const int64_t row = r0 + rs * RPS + sub;
        if (j == 0 && row < d_out) store(y, row, v);
      }
    }
  };

  // load cursor (li, lc, ls) runs one unit ahead of the compute cursor (ci, cc, cn)
  Src<RS> ls;
  int64_t li = w0;
  int lc = 0;
  if (active) setup(li, ls);
  int64_t ci = w0;
  int cc = 0;
  int cn = active ? ls.nchunk : 0;
  auto advance_load = [&]() {
    if (++lc == ls.nchunk) {
      lc = 0;
      li += W;
      if (li < nitems) setup(li, ls);
    }
  };
  // returns false when the wavefront's last unit has been reduced
  auto advance_compute = [&]() {
    if (++cc < cn) return true;
    finish(ci);
    ci += W;
    if (ci >= nitems) return false;
    cc = 0;
    cn = uniform_int(t.d_in[problem_of(ci)]) / kGroup / LPR;
    return true;
  };
  Chunk<1, RS> ca, cb;
  if constexpr (kLut) {
    // The first two units' loads are issued before the code table is written, so that the table's
    // 64 KB of LDS stores overlap their latency; every wavefront (idle ones too) writes its share
    // of the table and meets the barrier before any wavefront returns.
    if (active) {
      load(ls, lc, ca);
      advance_load();
      load(ls, lc, cb);
      if (li < nitems) advance_load();
    }
    for (int i = threadIdx.x; i < 256 * 64 / 4; i += kStreamThreads) {  // 4 copies of entry i / 16 per store
      const uint32_t v = lut_pair(i >> 4);
      reinterpret_cast<u32x4*>(lut)[i] = u32x4{v, v, v, v};
    }
    __syncthreads();
    if (!active) return;  // no barrier follows
    while (true) {
      asm volatile("" ::: "memory");
      compute(ca);
      if (!advance_compute()) break;
      load(ls, lc, ca);
      if (li < nitems) advance_load();
      asm volatile("" ::: "memory");
      compute(cb);
      if (!advance_compute()) break;
      load(ls, lc, cb);
      if (li < nitems) advance_load();
    }
  } else {
    // The loads are issued unconditionally: past the wavefront's last unit the cursor still holds
    // the last item, so a spare (valid, unused) unit is loaded.  Every reduction then has the same
    // number of loads after it, and the wait before it is a fixed count instead of a full drain.
    if (!active) return;  // no barrier follows
    load(ls, lc, ca);
    advance_load();
    while (true) {
      load(ls, lc, cb);
      if (li < nitems) advance_load();
      asm volatile("" ::: "memory");
      compute(ca);
      if (!advance_compute()) break;
      load(ls, lc, ca);
      if (li < nitems) advance_load();
      asm volatile("" ::: "memory");
      compute(cb);
      if (!advance_compute()) break;
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
                       dim3(kThreads), 0, s, x, static_cast<int>(m), packed, s16, d_out, d_in, y, ydt);
  } else if (waves1 >= 2 * 1024) {
    const int64_t waves = (d_out + 2 * RPS - 1) / (2 * RPS);
    hipLaunchKernelGGL((gemv_kernel<MT, LPR, 2>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                       dim3(kThreads), 0, s, x, static_cast<int>(m), packed, s16, d_out, d_in, y, ydt);
  } else {
    hipLaunchKernelGGL((gemv_kernel<MT, LPR, 1>), dim3(static_cast<unsigned>((waves1 + 3) / 4)),
                       dim3(kThreads), 0, s, x, static_cast<int>(m), packed, s16, d_out, d_in, y, ydt);
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

namespace w4q {
namespace {

// Workgroups of a kernel that fit on the device at once: compute units x resident workgroups per
// compute unit, queried once per device and kernel.
int resident_grid(const void* kernel, int slot, int threads = kThreads) {
  constexpr int kDevices = 64;
  static std::atomic<int> cache[kDevices][24];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kDevices) {
    const int v = cache[dev][slot].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess) return 0;
  const int v = cus * (per > 0 ? per : 1);
  if (dev < kDevices) cache[dev][slot].store(v, std::memory_order_relaxed);
  return v;
}

template <int LPR, int RS, bool kLut>
int launch_stream(const GroupArgs& a, int64_t items, int slot, hipStream_t s) {
  constexpr int nt = stream_threads<kLut>();
  auto* k = &gemv_stream_kernel<LPR, RS, kLut>;
  const int res = resident_grid(reinterpret_cast<const void*>(k), slot, nt);
  if (res <= 0) return W4Q_EHIP;
  const int64_t need = (items + nt / 64 - 1) / (nt / 64);
  const unsigned grid = static_cast<unsigned>(need < res ? need : res);
  hipLaunchKernelGGL(k, dim3(grid), dim3(nt), 0, s, a);
  return w4q_launch_status();
}

template <bool kLut>
int launch_stream_lpr(const GroupArgs& a, int64_t items, int lpr, hipStream_t s) {
  constexpr int base = kLut ? 0 : 7;  // resident-grid cache slots
  switch (lpr) {
    case 64: return launch_stream<64, 4, kLut>(a, items, base + 0, s);
    case 32: return launch_stream<32, 4, kLut>(a, items, base + 1, s);
    case 16: return launch_stream<16, 4, kLut>(a, items, base + 2, s);
    case 8: return launch_stream<8, 4, kLut>(a, items, base + 3, s);
    case 4: return launch_stream<4, 4, kLut>(a, items, base + 4, s);
    case 2: return launch_stream<2, 4, kLut>(a, items, base + 5, s);
    default: return launch_stream<1, 4, kLut>(a, items, base + 6, s);
  }
}

// lane split of a launch: the largest power of two (<= 64) dividing every group count
int chunk_lpr(const w4q_gemv_problem* probs, int cnt) {
  int lpr = 64;
  for (int i = 0; i < cnt; ++i)
    while ((probs[i].d_in / kGroup) % lpr != 0) lpr >>= 1;
  return lpr;
}

// items (4 row-steps of 64 / lpr rows) of problems [0, cnt)
int64_t chunk_items(const w4q_gemv_problem* probs, int cnt, int lpr) {
  const int rows_per_item = 4 * (64 / lpr);
  int64_t items = 0;
  for (int i = 0; i < cnt; ++i) items += (probs[i].d_out + rows_per_item - 1) / rows_per_item;
  return items;
}

// problems [0, cnt) of `probs` in one launch (sizes checked by w4q_gemv_group_fits).  Launches of
// at least 48 MB of codes whose items fill every wavefront of a resident grid convert codes through
// the LDS table (its 64 KB per workgroup are written once and amortised over many units); smaller
// ones take the byte-select conversion, whose workgroups start streaming at once.  (Measured per
// launch, 4096x4096 repeated: 5.4 us with the table, 4.0 us without; 24576x4096: 12.3 vs 13.9 us;
// all 252 linears of the 36-layer stack in 64-problem launches: 699 vs 836 us.)
int launch_group_chunk(const w4q_gemv_problem* probs, int cnt, int y_dtype, hipStream_t s) {
  GroupArgs a = {};
  const int lpr = chunk_lpr(probs, cnt);
  const int rows_per_item = 4 * (64 / lpr);
  int64_t items = 0, bytes = 0;
  for (int i = 0; i < cnt; ++i) {
    const w4q_gemv_problem& q = probs[i];
    a.x[i] = q.x;
    a.packed[i] = q.packed;
    a.s16[i] = q.scale_f16;
    a.y[i] = q.y;
    a.d_out[i] = static_cast<int>(q.d_out);
    a.d_in[i] = static_cast<int>(q.d_in);
    a.first[i] = static_cast<int>(items);
    items += (q.d_out + rows_per_item - 1) / rows_per_item;
    bytes += q.d_out * q.d_in / 2;
  }
  a.first[cnt] = static_cast<int>(items);
  a.n = cnt;
  a.y_dtype = y_dtype;
  if (bytes >= (int64_t(48) << 20) && items >= 4096) return launch_stream_lpr<true>(a, items, lpr, s);
  return launch_stream_lpr<false>(a, items, lpr, s);
}

}  // namespace
}  // namespace w4q

// 2..16 activation rows: one matrix-core launch.  A single row takes the stream kernel (as a
// one-problem group) when its sizes fit 32 bits, else the vector kernel.
int w4q_launch_gemv(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                    int64_t d_out, int64_t d_in, void* y, int y_dtype, hipStream_t s) {
  if (m >= 2 && m <= 16) {
    const int tiles = d_out < 8192 ? 1 : 2;
    const int64_t blocks = (d_out + 16 * tiles - 1) / (16 * tiles);
    if (blocks > 0x7FFFFFFF) return W4Q_EUNSUPPORTED;
    const bool vec = (d_in / kGroup) % kMmaBatch == 0;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kMmaWaves * 64);
    const int mr = static_cast<int>(m);
    // 16 wavefronts per workgroup (twice the loads in flight per compute unit) on long rows with
    // one tile per workgroup: d_in >= 8192 gives each wavefront two 8-group batches or more
    // (measured at 4096x12288, M = 2..8: 17.6 -> 15.5 us at M = 2; no gain at M = 16, and a loss
    // where the wavefronts get one batch each)
    if (tiles == 1 && d_in >= 8192 && m <= 8) {
      const dim3 block16(16 * 64);
      if (vec)
        hipLaunchKernelGGL((gemv_mma_kernel<true, 1, 16>), grid, block16, 0, s, x, mr, packed, s16, d_out, d_in, y,
                           y_dtype);
      else
        hipLaunchKernelGGL((gemv_mma_kernel<false, 1, 16>), grid, block16, 0, s, x, mr, packed, s16, d_out, d_in, y,
                           y_dtype);
      return w4q_launch_status();
    }
    if (vec && tiles == 2)
      hipLaunchKernelGGL((gemv_mma_kernel<true, 2>), grid, block, 0, s, x, mr, packed, s16, d_out, d_in, y, y_dtype);
    else if (vec)
      hipLaunchKernelGGL((gemv_mma_kernel<true, 1>), grid, block, 0, s, x, mr, packed, s16, d_out, d_in, y, y_dtype);
    else if (tiles == 2)
      hipLaunchKernelGGL((gemv_mma_kernel<false, 2>), grid, block, 0, s, x, mr, packed, s16, d_out, d_in, y, y_dtype);
    else
      hipLaunchKernelGGL((gemv_mma_kernel<false, 1>), grid, block, 0, s, x, mr, packed, s16, d_out, d_in, y, y_dtype);
    return w4q_launch_status();
  }
  // one activation row: the persistent stream kernel, or the plain vector kernel when the
  // stream's 32-bit offsets do not cover the shape
  const w4q_gemv_problem one = {x, packed, s16, y, d_out, d_in};
  if (d_out <= 0x7FFFFFFF && d_in <= (1 << 24) && w4q_gemv_group_fits(&one, 1))
    return launch_group_chunk(&one, 1, y_dtype, s);
  return launch_mt<1>(x, 1, packed, s16, d_out, d_in, y, y_dtype, s);
}

// Every launch's item count fits an int and every item's lane offsets fit 32 bits
// (rows_per_item * d_in / 2 < 2^32, which d_in <= 2^24 guarantees).
bool w4q_gemv_group_fits(const w4q_gemv_problem* probs, int n) {
  for (int b = 0; b < n; b += kMaxGroup) {
    const int cnt = n - b < kMaxGroup ? n - b : kMaxGroup;
    const int lpr = chunk_lpr(probs + b, cnt);
    for (int i = 0; i < cnt; ++i)
      if (probs[b + i].d_in / 2 * (4 * (64 / lpr)) > 0xFFFFFFFFll) return false;
    if (chunk_items(probs + b, cnt, lpr) > 0x7FFFFFFF) return false;
  }
  return true;
}

// One launch for up to kMaxGroup one-row products (any d_out, d_in % 32 == 0).
int w4q_launch_gemv_group(const w4q_gemv_problem* probs, int n, int y_dtype, hipStream_t s) {
  for (int b = 0; b < n; b += kMaxGroup) {
    const int rc = launch_group_chunk(probs + b, n - b < kMaxGroup ? n - b : kMaxGroup, y_dtype, s);
    if (rc != W4Q_OK) return rc;
  }
  return W4Q_OK;
}

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
// and the factor 8 is removed (exactly) after the row reduction.  The bias is 24/|q| times the
// signal, so the fp32 sum error stays near 2^-24 * 31 * sum|x| per group.  The next chunk's
// codes, scales and activations are loaded while the current chunk is being reduced.
#include "common.hpp"

namespace w4q {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kMask = 0x00780078u;  // mantissa bits 3..6 of each bf16 half
constexpr uint32_t kC0 = 0x43404340u;    // bf16 pair 2^7 with the nibble bias folded in
constexpr uint32_t kZero = 0x43404340u;  // code q = 0 (n = 8) in both halves

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

// 8 activations x[8b .. 8b+7] as 4 dwords (x0,x1)(x2,x3)(x4,x5)(x6,x7) -> the pairs
// (x0,x4)(x1,x5)(x2,x6)(x3,x7) that match the nibble pairs extracted below.
__device__ __forceinline__ void pair_x(const u32x4 d, uint32_t* p) {
  p[0] = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);
  p[1] = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);
  p[2] = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);
  p[3] = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);
}

// 8 two's-complement nibbles (one dword) -> 4 bf16 pairs (nibble i with i+4) holding
// 8 * (24 + q).  ((v >> s) & mask) ^ c0 moves a nibble to mantissa bits 3..6 and flips its top
// bit (two's complement -> offset binary n = q + 8) while inserting the exponent; the
// compiler emits one v_bitop3 per pair with mask in an SGPR and c0 in a VGPR.
__device__ __forceinline__ void codes_bf16(uint32_t v, uint32_t mask, uint32_t c0, uint32_t* c) {
  c[0] = ((v << 3) & mask) ^ c0;
  c[1] = ((v >> 1) & mask) ^ c0;
  c[2] = ((v >> 5) & mask) ^ c0;
  c[3] = ((v >> 9) & mask) ^ c0;
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
                                          void* __restrict__ y, int y_dtype, uint32_t mask, int64_t block) {
  constexpr int RPS = 64 / LPR;  // rows per row-step
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;
  const int j = lane % LPR;
  const int64_t wave = block * (kThreads / 64) + threadIdx.x / 64;
  const int64_t row0 = wave * (RPS * RS);
  if (row0 >= d_out) return;  // uniform per wavefront
  const int G = static_cast<int>(d_in / kGroup);
  const int nchunk = G / LPR;
  uint32_t c0 = kC0;
  asm volatile("" : "+v"(c0));  // keep the constant in a VGPR so v_bitop3 can take it

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
    // activations of this group, paired, plus the zero-code sum (same dot2 order as below)
    uint32_t xp[MT][16];
    float corr[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int b = 0; b < 4; ++b) pair_x(m < m_rows ? cur.xv[m][b] : u32x4{0u, 0u, 0u, 0u}, &xp[m][4 * b]);
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) a = dot2(xp[m][i], kZero, a);
      corr[m] = a;
    }
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      uint32_t cb[16];
      const uint32_t words[4] = {cur.code[rs].x, cur.code[rs].y, cur.code[rs].z, cur.code[rs].w};
#pragma unroll
      for (int b = 0; b < 4; ++b) codes_bf16(words[b], mask, c0, &cb[4 * b]);
      const float sc = f16_bits_to_f32(static_cast<uint16_t>(cur.sc[rs]));
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a = dot2(xp[m][i], cb[i], a);
        acc[rs][m] = __builtin_fmaf(sc, a - corr[m], acc[rs][m]);
      }
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
  // reduce the LPR lane partials of each row (fixed butterfly order); undo the factor 8
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const int64_t n = row0 + rs * RPS + sub;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[rs][m];
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      v *= 0.125f;
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
                                                        void* __restrict__ y, int y_dtype,
                                                        uint32_t mask) {
  gemv_body<MT, LPR, RS>(x, m_rows, packed, s16, d_out, d_in, y, y_dtype, mask, blockIdx.x);
}

// Many independent one-row products in one launch: workgroup b belongs to the problem p with
// first[p] <= b < first[p + 1] and works on that problem's rows as its workgroup b - first[p].
constexpr int kMaxGroup = 32;
constexpr int64_t kGroupGrid = 256 * 12;  // workgroups of the grouped launch
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
  uint32_t mask;
};

// (the grid is a fixed number of workgroups that walk the row blocks with a stride, so the
// wavefronts live long and keep loads in flight; problems are visited in order)
template <int LPR, int RS>
__global__ __launch_bounds__(kThreads) void gemv_group_kernel(const GroupArgs a) {
  int p = 0;
  for (int b = blockIdx.x; b < a.first[a.n]; b += gridDim.x) {
    while (p + 1 < a.n && b >= a.first[p + 1]) ++p;  // uniform
    gemv_body<1, LPR, RS>(a.x[p], 1, a.packed[p], a.s16[p], a.d_out[p], a.d_in[p], a.y[p], a.y_dtype,
                          a.mask, b - a.first[p]);
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
                       dim3(kThreads), 0, s, x, static_cast<int>(m), packed, s16, d_out, d_in, y, ydt, kMask);
  } else if (waves1 >= 2 * 1024) {
    const int64_t waves = (d_out + 2 * RPS - 1) / (2 * RPS);
    hipLaunchKernelGGL((gemv_kernel<MT, LPR, 2>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                       dim3(kThreads), 0, s, x, static_cast<int>(m), packed, s16, d_out, d_in, y, ydt, kMask);
  } else {
    hipLaunchKernelGGL((gemv_kernel<MT, LPR, 1>), dim3(static_cast<unsigned>((waves1 + 3) / 4)),
                       dim3(kThreads), 0, s, x, static_cast<int>(m), packed, s16, d_out, d_in, y, ydt, kMask);
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

// One launch for up to kMaxGroup one-row products (any d_out, d_in % 32 == 0).  Every problem
// uses the lane split of the largest power of two (<= 64) that divides all their group counts
// and four row-steps per wavefront.
int w4q_launch_gemv_group(const w4q_gemv_problem* probs, int n, int y_dtype, hipStream_t s) {
  for (int b = 0; b < n; b += kMaxGroup) {
    const int cnt = n - b < kMaxGroup ? n - b : kMaxGroup;
    GroupArgs a = {};
    int lpr = 64;
    for (int i = 0; i < cnt; ++i)
      while ((probs[b + i].d_in / kGroup) % lpr != 0) lpr >>= 1;
    const int rows_per_block = 4 * 4 * (64 / lpr);  // 4 wavefronts x 4 row-steps x rows per step
    int64_t blocks = 0;
    for (int i = 0; i < cnt; ++i) {
      const w4q_gemv_problem& q = probs[b + i];
      a.x[i] = q.x;
      a.packed[i] = q.packed;
      a.s16[i] = q.scale_f16;
      a.y[i] = q.y;
      a.d_out[i] = static_cast<int>(q.d_out);
      a.d_in[i] = static_cast<int>(q.d_in);
      a.first[i] = static_cast<int>(blocks);
      blocks += (q.d_out + rows_per_block - 1) / rows_per_block;
    }
    if (blocks > 0x7FFFFFFF) return W4Q_EUNSUPPORTED;
    a.first[cnt] = static_cast<int>(blocks);
    a.n = cnt;
    a.y_dtype = y_dtype;
    a.mask = kMask;
    // enough workgroups for every compute unit to hold a few, each walking many row blocks
    const dim3 grid(static_cast<unsigned>(blocks < kGroupGrid ? blocks : kGroupGrid));
    switch (lpr) {
      case 64: hipLaunchKernelGGL((gemv_group_kernel<64, 4>), grid, dim3(kThreads), 0, s, a); break;
      case 32: hipLaunchKernelGGL((gemv_group_kernel<32, 4>), grid, dim3(kThreads), 0, s, a); break;
      case 16: hipLaunchKernelGGL((gemv_group_kernel<16, 4>), grid, dim3(kThreads), 0, s, a); break;
      case 8: hipLaunchKernelGGL((gemv_group_kernel<8, 4>), grid, dim3(kThreads), 0, s, a); break;
      case 4: hipLaunchKernelGGL((gemv_group_kernel<4, 4>), grid, dim3(kThreads), 0, s, a); break;
      case 2: hipLaunchKernelGGL((gemv_group_kernel<2, 4>), grid, dim3(kThreads), 0, s, a); break;
      default: hipLaunchKernelGGL((gemv_group_kernel<1, 4>), grid, dim3(kThreads), 0, s, a); break;
    }
    const int rc = w4q_launch_status();
    if (rc != W4Q_OK) return rc;
  }
  return W4Q_OK;
}

// hessian.hip -- H = X^T X for bf16 calibration activations on the bf16 matrix cores.
//
// Method: blog "Opt.Gear-QAT: Preserving On-Device Performance with QAT", section 2 (the
// second-order output-reconstruction view from GPTQ; layer sensitivity from calibration
// inputs): for the objective of the model card's "Quantization Configuration",
// ||W X - Q(W) X||^2 is a quadratic form in the weight error with matrix X^T X.
//
// Only the 256x256 tiles on and above the diagonal are computed (the algorithmic work is the
// unique entries of the symmetric result); each value is written to both (i, j) and (j, i), so
// H is bitwise symmetric.
//
// Work split (stream-K): the (tile, 32-token stage) iterations of the whole triangle, tile-major,
// are cut into one contiguous range per workgroup, so every compute unit gets the same number of
// matrix-core steps whatever the tile count.  A tile whose stages are spread over several
// workgroups is finished by a second kernel that adds the partial tiles in the fixed order of
// their token ranges: the result does not depend on scheduling.  The partial tiles live in
// scratch memory the caller passes; with less scratch than the even split wants, the ranges are
// lengthened until their partial tiles fit, or become whole tiles (no scratch at all).
//
// Per workgroup: 8 wavefronts (two per SIMD) of 128x64 (4x2 v_mfma_f32_32x32x16_bf16 blocks),
// 32 tokens per stage, four LDS stage buffers.  Two wavefronts per SIMD because the transposing
// LDS reads below deliver almost twice the bytes per clock with two wavefronts per SIMD as with
// one (about 180 vs 100 B/clk per compute unit measured on gfx950), and because vector and LDS
// work of one wavefront only overlaps the matrix cores when it comes from another wavefront.  X is row-major [token][feature], the
// layout in which it is copied straight from memory into LDS by buffer loads to LDS (16 bytes
// per lane, no registers); the MFMA fragments, which want 8 consecutive tokens of one feature per
// lane, are then read with the transposing LDS read ds_read_b64_tr_b16.  Buffer loads past the
// end of X return zeros, which pads the token tail without any test in the loop.
#include "common.hpp"

#include <type_traits>

namespace w4q {
namespace {

constexpr int kThreads = 512;
constexpr int BT = 256;                // tile edge in features
constexpr int BK = 32;                 // tokens per stage
constexpr int NBUF = 4;                // LDS stage buffers: loads run NBUF - 1 stages ahead
constexpr int kTileElems = BT * BT;    // floats per partial tile
constexpr int kMinChunk = 16;          // stages per workgroup before more workgroups are used
constexpr int kMaxBlocks = 256;        // one workgroup per compute unit
constexpr int kStageBytes = 2 * BK * BT * 2;    // I and J panels, bf16: 32 KB
constexpr int kLoadsPerWave = kStageBytes / 1024 / 8;  // 1 KB per load instruction: 4

// LDS stage layout: panel p (I = 0, J = 1), token t, 16-byte chunk position cp (32 per token row
// of 256 features).  Chunk c (features 8c .. 8c + 7) of token t sits at position c ^ swz(t % 4).
// A transposing read of 16 lanes covers 4 consecutive tokens x 2 chunks (and a pair of 16-lane
// groups 4 tokens x 4 chunks); with these four masks the 16 lanes hit 8 distinct 16-byte bank
// slots modulo 128 bytes, and the 32 lanes 16 distinct slots modulo 256 bytes.
__device__ __forceinline__ int swz(int t) { return (0xCA60 >> (4 * (t & 3))) & 15; }  // 0, 6, 10, 12

// upper-triangle tile t, numbered row-major over ti <= tj
__device__ __forceinline__ void tile_coords(int t, int nt, int& ti, int& tj) {
  int rem = t, i = 0;
  while (rem >= nt - i) {
    rem -= nt - i;
    ++i;
  }
  ti = i;
  tj = i + rem;
}

// Store one 32x32 accumulator block whose top-left entry is (row0, col0), row0 <= col0 (both
// wave-uniform), into both triangles.  Accumulator layout: lane l, register r -> row
// 8(r/4) + 4(l/32) + r%4, column l%32; registers 4a..4a+3 are four consecutive rows, i.e. four
// consecutive entries of one row of the mirrored block, written with one 16-byte store.
__device__ __forceinline__ void store_block(float* __restrict__ h, int d, int row0, int col0, const f32x16& v,
                                            int accumulate, int lane) {
  const int c = lane & 31;
  if (col0 + c >= d) return;
  float* __restrict__ hd = h + (int64_t)row0 * d + col0;  // direct block, row-major
  float* __restrict__ hm = h + (int64_t)col0 * d + row0;  // mirrored block
  const bool straddle = row0 == col0;                     // the block holds diagonal entries
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int r = 8 * a + 4 * (lane >> 5);
    if (row0 + r >= d) continue;  // d % 8 == 0: rows r .. r + 3 are all inside or all outside
    float o[4] = {v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]};
    if (!straddle) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (accumulate) o[q] += hd[(r + q) * d + c];
        hd[(r + q) * d + c] = o[q];
      }
      *reinterpret_cast<f32x4*>(hm + c * d + r) = f32x4{o[0], o[1], o[2], o[3]};
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (r + q > c) continue;
        float val = o[q];
        if (accumulate) val += hd[(r + q) * d + c];
        hd[(r + q) * d + c] = val;
        if (r + q != c) hm[c * d + r + q] = val;
      }
    }
  }
}

// partial-tile layout (per workgroup slot): wave w, block (i, j), register quad a, lane l ->
// float4 at ((w * 8 + i * 2 + j) * 4 + a) * 256 + 4 l; each store instruction writes 1 KB.
__device__ __forceinline__ int64_t part_off(int w, int i, int j, int a, int lane) {
  return (int64_t)(((w * 8 + i * 2 + j) * 4 + a) * 256 + 4 * lane);
}

#define W4Q_LDS4(p) ((__attribute__((address_space(3))) v4i16*)(p))

static_assert(kLoadsPerWave == 4, "one dma_x4 per stage and wave");

__global__ __launch_bounds__(kThreads, 1) void hessian_kernel(const uint16_t* __restrict__ x, int n_tok, int d,
                                                              float* __restrict__ h, int accumulate, int nt,
                                                              int ns, int total, int chunk, int nblk,
                                                              int per_xcd, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) uint16_t Ls[NBUF * kStageBytes / 2];

  // workgroups are dealt to the 8 XCDs round-robin; consecutive ranges (which share tiles and
  // hence I panels and partial tiles) go to the same XCD
  const int lb = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lb >= nblk) return;
  const int it_begin = lb * chunk;
  const int it_end = it_begin + chunk < total ? it_begin + chunk : total;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 2, wn = wid & 3;

  // load role: load q (0..3) of wave w fills the 1 KB of LDS at (4 w + q) KB: panel w / 4,
  // tokens 8 (w % 4) + 2 q + lane / 32, chunk position lane % 32
  const int ld_panel = wid >> 2;
  int ld_tok[kLoadsPerWave], ld_chunk[kLoadsPerWave];
#pragma unroll
  for (int q = 0; q < kLoadsPerWave; ++q) {
    ld_tok[q] = 8 * (wid & 3) + 2 * q + (lane >> 5);
    ld_chunk[q] = (lane & 31) ^ swz(ld_tok[q]);
  }
  const uint32_t lds_base = lds_addr(Ls);

  // read role (transposing reads): 16-lane group g = lane / 16, lane j = lane % 16 in it points
  // at token 8 (g / 2) + j / 4 (+ 4 for the second read) and at features 16 (g % 2) + 4 (j % 4)
  // of a 32-feature block; it receives feature 16 (g % 2) + j of four consecutive tokens
  const int rg = lane >> 4, rj = lane & 15;
  const int rtok = 8 * (rg >> 1) + (rj >> 2);
  const int rsw = swz(rj >> 2);
  const int rlo = 2 * (rg & 1) + ((rj >> 1) & 1);  // chunk within a 32-feature block
  const int rhalf = 8 * (rj & 1);                  // byte within the chunk
  // byte offset in a stage of the read for 32-feature block `blk` (0..7 of a panel)
  auto rd_off = [&](int panel, int blk) { return panel * (kStageBytes / 2) + rtok * 512 + 16 * ((4 * blk + rlo) ^ rsw) + rhalf; };

  const f32x16 zero16 = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f,
                         0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};

  int it = it_begin;
  while (it < it_end) {
    const int t = it / ns;
    const int s0 = it - t * ns;
    const int s1 = s0 + (it_end - it) < ns ? s0 + (it_end - it) : ns;
    int ti, tj;
    tile_coords(t, nt, ti, tj);
    const bool diag = ti == tj;

    // byte offsets of this lane's loads within a stage; features past d read into the next token
    // or past the end (zeros): they only feed entries that are never stored
    const int fbase = (ld_panel ? tj : ti) * BT;
    int voff[kLoadsPerWave];
#pragma unroll
    for (int q = 0; q < kLoadsPerWave; ++q) voff[q] = (ld_tok[q] * d + fbase + 8 * ld_chunk[q]) * 2;
    // on a diagonal tile the J panel is the I panel: its loads are switched off
    const bool ld_on = !(diag && ld_panel == 1);

    auto issue = [&](int s) {
      const int64_t tok0 = (int64_t)s * BK;
      // bytes from the stage start to the end of X; 0 (every load returns zeros without touching
      // memory) for stages outside this range
      const int bytes = (s < s1 && ld_on) ? (n_tok - static_cast<int>(tok0)) * d * 2 : 0;
      const v4i32 rs = buffer_rsrc(x + tok0 * d, bytes);
      const uint32_t m0 = lds_base + static_cast<uint32_t>(((s - s0) % NBUF) * kStageBytes + 4 * 1024 * wid);
      dma_x4(m0, rs, voff);
    };
    // wait for this wave's loads of the stage about to be used (the NBUF - 2 younger stages stay
    // in flight), then a barrier: the stage is in LDS for all wavefronts, and every wavefront is
    // done with the buffer the next issue overwrites
    auto stage_sync = [&]() {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoadsPerWave * (NBUF - 2)));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    f32x16 acc[4][2];
    const int bpanel = diag ? 0 : 1;  // B fragments come from the I panel on diagonal tiles
    // fragments of one 16-token step of stage s (transposing reads)
    struct Frag {
      bf16x8 a[4], b[2];
    };
    auto load = [&](int s, int kk, Frag& F) {
      const char* Lb = reinterpret_cast<const char*>(Ls) + ((s - s0) % NBUF) * kStageBytes + kk * 16 * 512;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const char* p = Lb + rd_off(0, 4 * wm + i);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(W4Q_LDS4(p));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(W4Q_LDS4(p + 4 * 512));
        F.a[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const char* p = Lb + rd_off(bpanel, 2 * wn + j);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(W4Q_LDS4(p));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(W4Q_LDS4(p + 4 * 512));
        F.b[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    // products of rows i0 .. i1 - 1 of the 4x2 blocks; `first` starts the sums from zero.  (On a
    // diagonal tile the wavefronts below the diagonal, wm = 1 with wn < 2, compute the mirror
    // of others' blocks as well, which keeps the loop free of branches around the
    // accumulators, but never store it.)
    auto mma = [&](const Frag& F, int i0, int i1, auto first) {
#pragma unroll
      for (int i = i0; i < i1; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (decltype(first)::value) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.a[i], F.b[j], zero16, 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.a[i], F.b[j], acc[i][j], 0, 0, 0);
          }
        }
    };
    // the barrier sits between the products of a stage's last step, so the matrix cores stay
    // busy while the wavefronts meet; right after it the first fragments of the next stage are
    // read (the instruction order around it is pinned)
    auto mid_sync = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      stage_sync();
      __builtin_amdgcn_sched_barrier(0);
    };
    static_assert(BK == 32, "two 16-token steps per stage");

    // stage s lives in buffer (s - s0) % NBUF; its loads are issued NBUF - 1 stages ahead, into
    // the buffer of stage s - 1, which every wavefront finished reading before the last barrier
    Frag F0, F1;
#pragma unroll
    for (int p = 0; p < NBUF - 1; ++p) issue(s0 + p);
    stage_sync();
    load(s0, 0, F0);
    issue(s0 + NBUF - 1);
    load(s0, 1, F1);
    mma(F0, 0, 4, std::true_type{});
    mma(F1, 0, 2, std::false_type{});
    mid_sync();
    load(s0 + 1, 0, F0);  // (past the range: a stale buffer, never used)
    mma(F1, 2, 4, std::false_type{});
    for (int s = s0 + 1; s < s1; ++s) {
      issue(s + NBUF - 1);
      load(s, 1, F1);
      mma(F0, 0, 4, std::false_type{});
      mma(F1, 0, 2, std::false_type{});
      mid_sync();
      load(s + 1, 0, F0);
      mma(F1, 2, 4, std::false_type{});
    }
    // every load of this range (including the empty ones past its end) has landed and every
    // wavefront is done with the buffers before the next range refills them
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    const bool work = !(diag && wm == 1 && wn < 2);
    if (work) {
      if (s0 == 0 && s1 == ns) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int row0 = ti * BT + wm * 128 + 32 * i;
            const int col0 = tj * BT + wn * 64 + 32 * j;
            if (row0 <= col0 && row0 < d) store_block(h, d, row0, col0, acc[i][j], accumulate, lane);
            asm volatile("" ::: "memory");  // one block at a time (bounds the live registers)
          }
      } else {
        // slot 0: the first tile of this range, slot 1: its last
        float* slot = ws + (int64_t)(2 * lb + (it == it_begin ? 0 : 1)) * kTileElems;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              *reinterpret_cast<f32x4*>(slot + part_off(wid, i, j, a, lane)) =
                  f32x4{acc[i][j][4 * a], acc[i][j][4 * a + 1], acc[i][j][4 * a + 2], acc[i][j][4 * a + 3]};
              asm volatile("" ::: "memory");
            }
      }
    }
    it += s1 - s0;
  }
}

// Tiles whose stages were spread over several workgroups: sum the partial tiles in the order of
// their token ranges (workgroup index), then store as the main kernel does.  One workgroup per
// (tile, 32x32 block row i, block column j) of every wavefront's 128x64 part.
__global__ __launch_bounds__(kThreads) void hessian_fixup_kernel(float* __restrict__ h, int d, int accumulate, int nt,
                                                                 int ns, int chunk, const float* __restrict__ ws) {
  const int t = blockIdx.x >> 3;
  const int i = (blockIdx.x >> 1) & 3, j = blockIdx.x & 1;
  const int first = static_cast<int>((int64_t)t * ns / chunk);
  const int last = static_cast<int>(((int64_t)t * ns + ns - 1) / chunk);
  if (first == last) return;  // written whole by the main kernel
  int ti, tj;
  tile_coords(t, nt, ti, tj);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 2, wn = wid & 3;
  if (ti == tj && wm == 1 && wn < 2) return;
  const int row0 = ti * BT + wm * 128 + 32 * i;
  const int col0 = tj * BT + wn * 64 + 32 * j;
  if (row0 > col0 || row0 >= d || col0 >= d) return;
  f32x16 v;
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = 0.0f;
  for (int b = first; b <= last; ++b) {
    // tile t is the first tile of workgroup b's range unless b started before it
    const int slot = 2 * b + ((int64_t)b * chunk >= (int64_t)t * ns ? 0 : 1);
    const float* p = ws + (int64_t)slot * kTileElems;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(p + part_off(wid, i, j, a, lane));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * a + e] += q[e];
    }
  }
  store_block(h, d, row0, col0, v, accumulate, lane);
}

// Schedule of one pass: stream-K ranges of `chunk` (tile, stage) iterations, one per workgroup,
// and the scratch their partial tiles need (two 256x256 fp32 slots per workgroup, only when some
// tile is split over workgroups).
struct Plan {
  int64_t nt, tiles, ns, total, chunk, nblk, per_xcd;
  bool split;
  size_t ws_need;
};

constexpr size_t kSlotPair = size_t(2) * kTileElems * sizeof(float);  // 512 KB per workgroup

void finish(Plan& p) {
  p.nblk = (p.total + p.chunk - 1) / p.chunk;
  p.split = p.nblk > 1 && p.chunk % p.ns != 0;
  p.ws_need = p.split ? size_t(p.nblk) * kSlotPair : 0;
  p.per_xcd = (p.nblk + 7) / 8;
}

// The fastest schedule whose scratch fits ws_bytes (SIZE_MAX: the fastest one).
Plan plan_pass(int64_t n_tok, int64_t d, size_t ws_bytes) {
  Plan p;
  p.nt = (d + BT - 1) / BT;
  p.tiles = p.nt * (p.nt + 1) / 2;
  p.ns = (n_tok + BK - 1) / BK;
  p.total = p.tiles * p.ns;
  // an even share of the stages for every compute unit, but at least kMinChunk stages (or a
  // whole tile) per workgroup: short ranges cost more in partial tiles than they gain.  Shares
  // shorter than 2 kMinChunk are lengthened to that while at least half the compute units stay
  // busy (measured: 4096 x 2048 tokens x features 60 -> 52 us)
  const int64_t min_chunk = p.ns < kMinChunk ? p.ns : kMinChunk;
  p.chunk = (p.total + kMaxBlocks - 1) / kMaxBlocks;
  if (p.chunk < 2 * kMinChunk && p.total / (2 * kMinChunk) >= kMaxBlocks / 2 && p.ns >= 2 * kMinChunk)
    p.chunk = 2 * kMinChunk;
  if (p.chunk < min_chunk) p.chunk = min_chunk;
  finish(p);
  if (p.ws_need <= ws_bytes) return p;
  // not enough scratch: the most workgroups whose partial tiles fit, or one whole tile per
  // workgroup (no scratch), whichever runs more workgroups
  const int64_t fit = static_cast<int64_t>(ws_bytes / kSlotPair);
  Plan q = p;
  q.chunk = q.ns;
  finish(q);
  if (fit >= 2) {
    Plan r = p;
    r.chunk = (r.total + fit - 1) / fit;
    finish(r);
    if (r.ws_need <= ws_bytes && r.nblk > q.nblk) return r;
  }
  return q;
}

// One pass over at most 2^31 - 1 bytes of X (32-bit buffer offsets).
int launch_pass(const uint16_t* x, int64_t n_tok, int64_t d, float* h, int accumulate, void* ws_ptr,
                size_t ws_bytes, hipStream_t s) {
  const Plan p = plan_pass(n_tok, d, ws_ptr != nullptr ? ws_bytes : 0);
  if (p.total > 0x3FFFFFFF) return W4Q_EUNSUPPORTED;
  float* ws = p.split ? static_cast<float*>(ws_ptr) : nullptr;
  hipLaunchKernelGGL(hessian_kernel, dim3(static_cast<unsigned>(8 * p.per_xcd)), dim3(kThreads), 0, s, x,
                     static_cast<int>(n_tok), static_cast<int>(d), h, accumulate, static_cast<int>(p.nt),
                     static_cast<int>(p.ns), static_cast<int>(p.total), static_cast<int>(p.chunk),
                     static_cast<int>(p.nblk), static_cast<int>(p.per_xcd), ws);
  int rc = w4q_launch_status();
  if (p.split && rc == W4Q_OK) {
    hipLaunchKernelGGL(hessian_fixup_kernel, dim3(static_cast<unsigned>(8 * p.tiles)), dim3(kThreads), 0, s, h,
                       static_cast<int>(d), accumulate, static_cast<int>(p.nt), static_cast<int>(p.ns),
                       static_cast<int>(p.chunk), ws);
    rc = w4q_launch_status();
  }
  return rc;
}

// tokens per pass: whole tokens within 32-bit buffer offsets
int64_t pass_tokens(int64_t d) { return 0x7FFFFFFF / (2 * d); }

}  // namespace
}  // namespace w4q

using namespace w4q;

size_t w4q_hessian_workspace(int64_t n_tok, int64_t d) {
  const int64_t max_tok = pass_tokens(d);
  const int64_t first = n_tok < max_tok ? n_tok : max_tok;
  const int64_t last = n_tok % max_tok == 0 ? first : n_tok % max_tok;
  const size_t a = plan_pass(first, d, SIZE_MAX).ws_need, b = plan_pass(last, d, SIZE_MAX).ws_need;
  return a > b ? a : b;
}

int w4q_launch_hessian(const uint16_t* x, int64_t n_tok, int64_t d, float* h, int accumulate,
                       void* ws, size_t ws_bytes, hipStream_t s) {
  // X is taken in passes of whole tokens that fit 32-bit buffer offsets; later passes add on
  // (stream order lets every pass reuse the same scratch)
  const int64_t max_tok = pass_tokens(d);
  for (int64_t t0 = 0; t0 < n_tok; t0 += max_tok) {
    const int64_t n = n_tok - t0 < max_tok ? n_tok - t0 : max_tok;
    const int rc = launch_pass(x + t0 * d, n, d, h, t0 == 0 ? accumulate : 1, ws, ws_bytes, s);
    if (rc != W4Q_OK) return rc;
  }
  return W4Q_OK;
}

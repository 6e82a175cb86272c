/*
 * w4a16q.h -- C ABI of the W4A16 group-wise quantization core for AMD gfx950 (MI355X).
 *
 * The method (symmetric INT4 weights, zero-point 0, one scale per group of 32 weights along
 * the input dimension, 16-bit activations) is the one described on these pages:
 *   [card]  model card "Opt.Gear-1B-qat-int4-per-channel-unquantized", sections
 *           "QAT Highlights" and "Quantization Configuration" (objective
 *           Delta* = argmin_Delta || W X - Q_Delta(W) X ||_F^2).
 *   [blog]  "Opt.Gear-QAT: Preserving On-Device Performance with QAT", sections
 *           "Quantization parameters of Opt.Gear-1B", "1. Quantization scale is important",
 *           "2. Hessian-based scale initialize", "3. LSQ-based QAT", "Conclusion".
 *   [blog-ko] the Korean edition of the same post, whose configuration table (group size 32)
 *           and role table survive intact.
 *
 * Common conventions for every entry point:
 *   - Tensors are caller-owned DEVICE memory, row-major, contiguous.  Every call only
 *     enqueues work on `stream` (0 = the legacy default stream) and returns; the library never
 *     synchronises.  Results are valid once the caller has synchronised that stream.  The
 *     library allocates nothing except one 128 MB device scratch buffer per device (partial
 *     tiles of quant_hessian, w4a16_gemm_dq, and w4a16_gemm when m > 16 runs the split-scale
 *     tiled kernel), made by the first such call on the device and kept until the process
 *     ends; the work of those calls on one device is serialised on it (a later call's stream
 *     waits for an event recorded after the earlier call's kernels).
 *   - Weights W are fp32 [d_out][d_in]; a group is 32 consecutive weights of one row along
 *     d_in, so d_in must be a positive multiple of 32 (W4Q_GROUP).  G = d_in / 32 groups/row.
 *   - Codes are integers in [-8, 7] (W4Q_QMIN..W4Q_QMAX).  code(w, D) is the code c that
 *     minimises |w - c*D| for the exact real quotient, ties going to the even code; this equals
 *     clamp(round_half_even(w / D), -8, 7).  For D == 0 the code is 0.
 *   - bf16 / fp16 values are passed as their raw 16-bit patterns (uint16_t).
 *   - Return value: W4Q_OK (0) or a negative status.  Argument errors are detected on the host
 *     before anything is enqueued.  W4Q_EHIP means a HIP launch error was reported; an error
 *     raised by a kernel during execution surfaces at the caller's next synchronisation.
 *   - Calls that touch disjoint outputs may run concurrently on different streams.
 */
#ifndef W4A16Q_H
#define W4A16Q_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4Q_GROUP 32  /* weights per quantization group ([blog-ko] configuration table) */
#define W4Q_QMIN (-8) /* symmetric signed INT4, zero-point fixed at 0 ([card] configuration) */
#define W4Q_QMAX 7    /* number of positive quantization levels ([blog] section 3) */
#define W4Q_MAX_CAND 255

enum w4q_status {
  W4Q_OK = 0,
  W4Q_EINVAL = -1,      /* null pointer, bad enum value, n_cand outside [1, 255] */
  W4Q_ESHAPE = -2,      /* non-positive size, d_in % 32 != 0, ldh < d_in, size overflow */
  W4Q_EALIGN = -3,      /* a pointer lacks the alignment stated for it below */
  W4Q_EUNSUPPORTED = -4,/* a size beyond what the kernels support (stated per call) */
  W4Q_EHIP = -5         /* the HIP runtime reported an error at launch */
};

/* Human-readable text for a status code (static storage, never NULL). */
const char* w4q_status_string(int status);

/* Library version as an integer, major * 10000 + minor * 100 + patch. */
int w4q_version(void);

/*
 * quant_hessian -- second-order statistics of the calibration activations.
 * [blog] section 2: layer sensitivity is estimated from calibration inputs in the
 * second-order output-reconstruction view taken from GPTQ; for the objective of [card]
 * "Quantization Configuration", ||W X - Q(W) X||^2 = sum over rows of e^T H e with H = X^T X.
 *
 *   x        bf16 [n_tok][d] calibration activations (tokens x input features). 16-B aligned.
 *   h        fp32 [d][d] output, H[i][j] = sum_t x[t][i] * x[t][j], unnormalised.
 *            H is written exactly symmetric (bitwise).  16-B aligned.
 *   accumulate  0: H = X^T X.   1: H += X^T X (H must hold a symmetric matrix on entry).
 *   Products bf16 x bf16 are exact in fp32; sums are accumulated in fp32 on the matrix cores.
 *   Limits: 1 <= n_tok, 1 <= d <= 65536, d % 8 == 0 (else W4Q_ESHAPE).
 */
int quant_hessian(const uint16_t* x, int64_t n_tok, int64_t d, float* h, int accumulate,
                  hipStream_t stream);

/*
 * quant_scale_search -- Hessian-weighted choice of one scale per group.
 * [card] "Quantization Configuration": the scale of each group is the minimiser of
 * ||W X - Q_Delta(W) X||_F^2; [blog] section 2 uses it in place of the max-based scale.
 * Read per group (the groups become independent): for row r, group g with weights
 * w = W[r][32g .. 32g+31] and the 32x32 diagonal block Hg = H[32g.., 32g..]:
 *   amax    = max_i |w_i|
 *   Delta_k = fp16_RNE( fl32( fl32(alpha[k] * amax) / 7 ) ), k = 0 .. n_cand-1
 *             (alpha = 1 gives the max-based scale; fp16 rounding puts every candidate on
 *             the deployed fp16 scale grid, so search, export and GEMM share one grid)
 *   e       = w - Delta_k * code(w, Delta_k)
 *   obj_k   = e^T Hg e
 *   idx     = the first k with the smallest obj_k.
 *
 *   w        fp32 [d_out][d_in], 16-B aligned.
 *   h        fp32 [d_in][ldh]; only the 32x32 diagonal blocks are read, and each block is
 *            taken to be symmetric (its upper triangle, diagonal included, is read).
 *   alpha    fp32 [n_cand] DEVICE array of candidate multipliers (> 0, finite).
 *   scale    fp32 [d_out][G] out: Delta_idx (an fp16-representable value).
 *   idx      uint8 [d_out][G] out: chosen candidate index.
 *   obj      fp32 [d_out][G] out or NULL: objective of the chosen candidate.
 *   obj_all  fp32 [d_out][G][n_cand] out or NULL: objective of every candidate.
 *   Objectives are scored in fp32; every group whose two best fp32 scores lie within a
 *   relative 1e-5 of each other is re-scored in fp64 before the choice is made.
 *   Precondition (not checked on the device): amax * alpha / 7 <= 65504.
 */
int quant_scale_search(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
                       const float* alpha, int n_cand, float* scale, uint8_t* idx, float* obj,
                       float* obj_all, hipStream_t stream);

/*
 * quant_pack -- export onto the deployment INT4 grid with the given scales.
 * [card] "QAT Highlights" and "Quickstart": the same grid is used at initialisation, QAT
 * and final conversion; [blog] "Conclusion": same symmetric group-32 grid at export.
 *   s16 = fp16_RNE(scale);  q = code(w, s16);  byte j of a packed row holds
 *   (q[2j] & 0xF) | (q[2j+1] & 0xF) << 4  (two's-complement nibbles, low nibble = even k).
 *
 *   w         fp32 [d_out][d_in] (finite), 16-B aligned.    scale  fp32 [d_out][G] (>= 0, finite).
 *   packed    uint8 [d_out][d_in/2] out, 16-B aligned.
 *   scale_f16 fp16 bits [d_out][G] out.
 */
int quant_pack(const float* w, const float* scale, int64_t d_out, int64_t d_in, uint8_t* packed,
               uint16_t* scale_f16, hipStream_t stream);

/*
 * lsq_fwd -- LSQ fake-quantisation forward pass.
 * [blog] section 3: the forward pass emulates the deployment symmetric INT4 grid with a
 * learnable step size Delta per group.
 *   w_hat[r][k] = fl32( Delta * code(w[r][k], Delta) ),  Delta = scale[r][k/32] (fp32, > 0).
 *   w, w_hat fp32 [d_out][d_in], 16-B aligned;  scale fp32 [d_out][G].
 */
int lsq_fwd(const float* w, const float* scale, int64_t d_out, int64_t d_in, float* w_hat,
            hipStream_t stream);

/*
 * lsq_bwd -- straight-through / LSQ backward pass.
 * [blog] section 3: round is bypassed with a straight-through estimator; the loss gradient
 * also reaches the step size, normalised by the group's element count and the number of
 * positive levels.  With G = dL/dw_hat, Delta = scale[r][g], q = code(w, Delta):
 *   m        = 1 if -8*Delta <= w <= 7*Delta else 0        (inclusive bounds)
 *   grad_w   = G * m
 *   f        = q - (w / Delta) * m
 *   grad_scale_out[r][g] = grad_scale * sum_{k in group} G_k * f_k
 * grad_scale is the normalisation factor, e.g. 1/sqrt(32 * 7) for the LSQ convention.
 *   w, grad_w_hat, grad_w fp32 [d_out][d_in] (16-B aligned); scale, grad_scale_out fp32
 *   [d_out][G];  w_hat: NULL, or fp32 [d_out][d_in] that also receives lsq_fwd's output.
 *   grad_scale_out is reduced in fp32 in a fixed order (run-to-run deterministic).
 */
int lsq_bwd(const float* w, const float* scale, const float* grad_w_hat, int64_t d_out,
            int64_t d_in, float grad_scale, float* grad_w, float* grad_scale_out, float* w_hat,
            hipStream_t stream);

/*
 * w4a16_gemm -- deployment W4A16 product on packed codes.
 * [card] intro and configuration: INT4 weights with 16-bit activations; speed is set by
 * weight memory, bandwidth and the kernels of the accelerator.
 *   w_hat[n][k] = fp32(scale_f16[n][k/32]) * q[n][k]   (exact in fp32)
 *   y[m][n]     = sum_k x[m][k] * w_hat[n][k]          (fp32 accumulation)
 *   x         bf16 [m][d_in], 16-B aligned.
 *   packed    uint8 [d_out][d_in/2] as written by quant_pack, 16-B aligned.
 *   scale_f16 fp16 bits [d_out][G], finite (an infinite scale gives undefined outputs).
 *   y         [m][d_out], fp32 (y_dtype 0) or bf16 RNE of the fp32 result (y_dtype 1).
 *   m >= 1.  Small m (<= 16) streams the packed weights once (bandwidth bound): m = 1 on the
 *   vector ALUs, 2..16 on the bf16 matrix cores; larger m is a tiled product on the matrix
 *   cores.  On the matrix cores the weights enter the products unrounded: either the codes
 *   enter as exact small bf16 integers and the fp32 scale is applied once per group to the
 *   group's partial products, or (shapes with few output tiles, d_in % 256 == 0) each weight
 *   is split into two bf16-exact parts, scale_hi * q + scale_lo * q, with scale_hi the fp16
 *   scale rounded to 5 significant bits.  Either way only the fp32 summation order differs
 *   from the definition above.
 */
int w4a16_gemm(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* scale_f16,
               int64_t d_out, int64_t d_in, void* y, int y_dtype, hipStream_t stream);

/*
 * w4a16_gemm_dq -- the same product with the weights dequantized to the 16-bit activation
 * format before the product ([card] W4A16: INT4 weights, 16-bit activations; the matrix cores
 * take bf16 operands):
 *   w_hat[n][k] = bf16_RNE(fp32(scale_f16[n][k/32]) * q[n][k])
 *   y[m][n]     = sum_k x[m][k] * w_hat[n][k]          (fp32 accumulation)
 * Arguments, layouts and y_dtype as for w4a16_gemm.  The weights are formed in registers and
 * go straight into the bf16 matrix-core products (no per-group scaling step); any m >= 1 runs
 * on the matrix cores.  d_in must be a multiple of 256 and d_out * d_in / 2 below 2^31 (else
 * W4Q_EUNSUPPORTED).
 */
int w4a16_gemm_dq(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* scale_f16,
                  int64_t d_out, int64_t d_in, void* y, int y_dtype, hipStream_t stream);

/*
 * w4a16_gemv_grouped -- many independent one-row W4A16 products (decode: one token through
 * several linears, e.g. the q/k/v or gate/up projections that share an input, or a whole
 * decoder's linears) in as few launches as possible: one launch per 64 problems.  Each problem
 * is the product of w4a16_gemm with m = 1 and the same arithmetic (exact weights s16 * q, fp32
 * accumulation); only the split of the row reduction over lanes may differ from other launches,
 * so results agree with them to fp32 rounding, not bitwise.
 *   problems   HOST array of n_problems descriptors; each x (bf16 [d_in], 16-B aligned),
 *              packed ([d_out][d_in/2], 16-B aligned), scale_f16 ([d_out][d_in/32]) and
 *              y ([d_out], fp32 or bf16 by y_dtype) is device memory as for w4a16_gemm.
 *   n_problems >= 0 (0 enqueues nothing).  Per problem d_out <= 2^31 - 1 and d_in <= 2^24
 *              (W4Q_EUNSUPPORTED otherwise).
 * Problems may share inputs; outputs must not overlap.  Argument errors (including
 * W4Q_EUNSUPPORTED) are reported before anything is enqueued.  The problem table is read
 * during the call only; the device memory it points to must stay valid until the stream
 * reaches the launch.  No scratch memory is used.
 */
typedef struct w4q_gemv_problem {
  const uint16_t* x;
  const uint8_t* packed;
  const uint16_t* scale_f16;
  void* y;
  int64_t d_out;
  int64_t d_in;
} w4q_gemv_problem;

int w4a16_gemv_grouped(const w4q_gemv_problem* problems, int n_problems, int y_dtype,
                       hipStream_t stream);

/*
 * Diagnostics (not part of the quantization path): measured peaks that rooflines are quoted
 * against besides the chip's nominal ones.
 *   w4q_probe_read       streams `bytes` (a multiple of 16, >= 16) of the 16-B aligned device
 *                        buffer `buf` once with 16-byte loads, non-temporal if nontemporal is 1
 *                        (0: ordinary loads, which also fill the caches); sink is device memory
 *                        of W4Q_PROBE_SINK_WORDS words, written at most at a few words.
 *   w4q_probe_mfma_bf16  runs `iters` (1 .. 2^24) rounds of 16 independent 32x32x16 bf16
 *                        matrix-core products on every wavefront (one per SIMD); sink is device
 *                        memory of W4Q_PROBE_SINK_WORDS floats; *flop (host, nullable) receives
 *                        the flop count of the launch.
 * Both enqueue one kernel on `stream` and return W4Q_EINVAL for bad arguments.
 */
#define W4Q_PROBE_SINK_WORDS 65536
int w4q_probe_read(const void* buf, int64_t bytes, int nontemporal, uint32_t* sink, hipStream_t stream);
int w4q_probe_mfma_bf16(float* sink, int64_t iters, double* flop, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* W4A16Q_H */

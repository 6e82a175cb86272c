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
 *     synchronises, allocates nothing and keeps no mutable state between calls.  Results are
 *     valid once the caller has synchronised that stream.
 *   - Scratch: quant_hessian, w4a16_gemm and w4a16_gemm_dq split output tiles over workgroups
 *     and keep the partial tiles in a caller-owned device workspace (workspace,
 *     workspace_bytes): NULL with 0 bytes, or 256-B aligned memory (W4Q_EINVAL for NULL with a
 *     non-zero size, W4Q_EALIGN if misaligned).  The matching *_workspace_size call returns the
 *     bytes the fastest schedule uses; with less, the call runs a schedule whose partial tiles
 *     fit (down to none: no scratch at all, fewer workgroups on small problems), with the same
 *     arithmetic up to the fp32 summation order.  The workspace is in use from the call until
 *     the stream has run its work: calls that may overlap (different streams, graph replays)
 *     need distinct workspaces.  The calls can be captured in HIP graphs (no allocation and no
 *     memset inside).
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
 *   workspace, workspace_bytes  caller-owned scratch (see the conventions above).
 *   Products bf16 x bf16 are exact in fp32; sums are accumulated in fp32 on the matrix cores.
 *   Limits: 1 <= n_tok, 1 <= d <= 65536, d % 8 == 0 (else W4Q_ESHAPE).
 */
int quant_hessian(const uint16_t* x, int64_t n_tok, int64_t d, float* h, int accumulate,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Scratch bytes of quant_hessian's fastest schedule for this shape (0: none), in *bytes (host).
 * Argument errors as for quant_hessian.  At most 128 MB. */
int quant_hessian_workspace_size(int64_t n_tok, int64_t d, size_t* bytes);

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
 *   h        fp32 [d_in][ldh], 16-B aligned, ldh >= d_in and a multiple of 4; only the 32x32
 *            diagonal blocks are read, all 32x32 entries of each (the form e^T Hg e uses both
 *            triangles, so a caller passing a triangle-only H gets wrong scores).
 *   alpha    fp32 [n_cand] DEVICE array of candidate multipliers (> 0, finite).
 *   scale    fp32 [d_out][G] out: Delta_idx (an fp16-representable value).
 *   idx      uint8 [d_out][G] out: chosen candidate index.
 *   obj      fp32 [d_out][G] out or NULL: objective of the chosen candidate.
 *   obj_all  fp32 [d_out][G][n_cand] out or NULL: objective of every candidate.
 *   Objectives are first scored with fp32-level error, each with an error radius
 *   2^-18 * |e|^T |Hg| |e|.  A group is re-scored in fp64 (the candidates whose interval
 *   reaches below the best one's; all of them when obj_all is requested) unless the best
 *   interval lies below every other and the reported objectives' radii are below 9e-6 of
 *   them.  So the chosen index is the exact first minimum up to fp64 rounding, and every
 *   reported objective is within 1e-5 relative of e^T Hg e.
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
 * lsq_adam_step -- one fused QAT optimisation step for one linear.
 * [blog] section 3: the weights and the step sizes are optimised jointly (the gradient reaches
 * the step through the LSQ estimator); [card] "QAT Highlights": the forward emulates the
 * deployment grid.  In one pass over W: the gradients of lsq_bwd (G = dL/dw_hat, D = the group's
 * fp32 step), then, in fp32 in this order, with hp's bias corrections c1 = 1 - beta1^t and
 * c2 = 1 - beta2^t of step t:
 *   g_w = G * m (STE mask)          m_w = beta1 m_w + (1 - beta1) g_w
 *                                    v_w = beta2 v_w + (1 - beta2) g_w^2
 *   w   = w - lr_w ((m_w / c1) / (sqrt(v_w / c2) + eps) + weight_decay w)
 *   ds  = grad_scale * sum_group G f  (as lsq_bwd)
 *   m_s = beta1 m_s + (1 - beta1) ds,  v_s = beta2 v_s + (1 - beta2) ds^2
 *   D   = max(D - lr_s (m_s / c1) / (sqrt(v_s / c2) + eps), scale_min)
 * Division and square root are correctly rounded.  The mask and the codes use the step and
 * weights before the update.
 *   w, m_w, v_w          fp32 [d_out][d_in] in/out (updated in place), 16-B aligned.
 *   scale, m_s, v_s      fp32 [d_out][G] in/out (updated in place).
 *   grad_w_hat           fp32 [d_out][d_in], 16-B aligned.
 *   hp                   HOST pointer: 0 <= beta < 1, eps > 0, 0 < c <= 1, lr >= 0,
 *                        weight_decay >= 0, scale_min > 0, all finite (else W4Q_EINVAL).
 *   grad_scale_out       fp32 [d_out][G] out or NULL: ds.
 *   w_hat_next           fp32 [d_out][d_in] out or NULL (16-B aligned): D_new * code(w_new,
 *                        D_new), the next step's forward.
 * Outputs must not overlap the inputs except the in/out pairs named above.
 */
typedef struct w4q_adam_params {
  float lr_w, lr_s;       /* learning rates of the weights and of the steps */
  float beta1, beta2, eps;
  float weight_decay;     /* decoupled, on the weights only */
  float bias_c1, bias_c2; /* 1 - beta1^t, 1 - beta2^t for step t >= 1 */
  float scale_min;        /* lower bound kept on every step */
} w4q_adam_params;

int lsq_adam_step(float* w, float* scale, const float* grad_w_hat, int64_t d_out, int64_t d_in,
                  float grad_scale, float* m_w, float* v_w, float* m_s, float* v_s,
                  const w4q_adam_params* hp, float* grad_scale_out, float* w_hat_next,
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
               int64_t d_out, int64_t d_in, void* y, int y_dtype, void* workspace,
               size_t workspace_bytes, hipStream_t stream);

/* Scratch bytes of w4a16_gemm's fastest schedule (0: none; the split-weight tiled kernel for
 * m > 16 with fewer output tiles than compute units is the only user; without its full scratch
 * the per-group kernel runs), in *bytes (host).  At most 128 MB. */
int w4a16_gemm_workspace_size(int64_t m, int64_t d_out, int64_t d_in, size_t* bytes);

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
                  int64_t d_out, int64_t d_in, void* y, int y_dtype, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/* Scratch bytes of w4a16_gemm_dq's fastest schedule (0: none), in *bytes (host).  At most
 * 128 MB. */
int w4a16_gemm_dq_workspace_size(int64_t m, int64_t d_out, int64_t d_in, size_t* bytes);

/*
 * w4a16_gemm_dq_noalloc -- w4a16_gemm_dq for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * product, kernels and arguments, without the workspace arguments.  Its scratch is a static
 * device array of 128 MB inside the library (the most any w4a16_gemm_dq schedule uses), which
 * every GPU the library runs on holds until the process ends; its address is looked up once per
 * device (the stream's device) and nothing is allocated.  Sizes whose fastest schedule would
 * need more than the array are refused with W4Q_EUNSUPPORTED.  All calls on one GPU share the
 * array: calls that overlap on one GPU (different streams, a graph replay beside a direct
 * call) race on it and give undefined results; calls in stream order on one stream are safe.
 */
int w4a16_gemm_dq_noalloc(const uint16_t* x, int64_t m, const uint8_t* packed,
                          const uint16_t* scale_f16, int64_t d_out, int64_t d_in, void* y,
                          int y_dtype, hipStream_t stream);

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

/* ------------------------------------------------------------------ per-channel variant
 * One scale per output row, the whole row being the group ([card] intro and "Quickstart":
 * the per-channel symmetric INT4 checkpoint).  Codes, nibble layout and the exact-quotient
 * code rule are those above; scales are fp32 [d_out] (search, LSQ) or fp16 bits [d_out]
 * (export, product).
 *
 * quant_scale_search_pc -- for row r with w = W[r][:] and the full H:
 *   amax = max_i |w_i|;  Delta_k = fp16_RNE(fl32(fl32(alpha[k] * amax) / 7));
 *   e = w - Delta_k * code(w, Delta_k);  obj_k = e^T H e;  idx = the first k with the smallest obj_k.
 *   Every e and every product and sum is fp64 (fp64 matrix cores), so the index is the exact
 *   first minimum up to fp64 rounding.  h: fp32 [d_in][ldh], all d_in x d_in entries read
 *   (16-B aligned, ldh >= d_in, ldh % 4 == 0).  scale fp32 [d_out] out, idx uint8 [d_out] out,
 *   obj fp32 [d_out] out or NULL, obj_all fp32 [d_out][n_cand] out or NULL.  No scratch.
 *   Precondition (not checked on the device): amax * alpha / 7 <= 65504.
 *
 * per_channel_workspace_size -- bytes of the workspace the four calls below take for an
 *   m x d_in activation (m = 1 for the calls without one): d_out x G steps, d_out x G partial
 *   sums, and the group product's workspace.  The calls broadcast the row's scale to the row's
 *   groups in the workspace and run the group-32 kernels: the codes, w_hat and dW are the same
 *   operations, the product differs only in summation order.  workspace: 256-B aligned, at least
 *   that size (W4Q_EINVAL if smaller or NULL, W4Q_EALIGN if misaligned).
 * quant_pack_pc   -- packed as quant_pack; scale_f16 [d_out] out = fp16_RNE(scale).
 * lsq_fwd_pc      -- w_hat = fl32(scale[r] * code(w, scale[r])).
 * lsq_bwd_pc      -- dW as lsq_bwd; grad_scale_out[r] = grad_scale * sum over the row of
 *                    G * (q - (w / Delta) m) (the group partial sums added in group order in fp64);
 *                    pass grad_scale = 1 / sqrt(d_in * 7) for the LSQ normalisation of a row.
 * w4a16_gemm_pc   -- y = x W_hat^T with W_hat[n][k] = fp16(scale_f16[n]) * q[n][k]; w_mode 0 as
 *                    w4a16_gemm (exact weights), 1 as w4a16_gemm_dq (bf16-dequantized weights).
 */
int quant_scale_search_pc(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
                          const float* alpha, int n_cand, float* scale, uint8_t* idx, float* obj,
                          float* obj_all, hipStream_t stream);
int per_channel_workspace_size(int64_t m, int64_t d_out, int64_t d_in, size_t* bytes);
int quant_pack_pc(const float* w, const float* scale, int64_t d_out, int64_t d_in, uint8_t* packed,
                  uint16_t* scale_f16, void* workspace, size_t workspace_bytes, hipStream_t stream);
int lsq_fwd_pc(const float* w, const float* scale, int64_t d_out, int64_t d_in, float* w_hat,
               void* workspace, size_t workspace_bytes, hipStream_t stream);
int lsq_bwd_pc(const float* w, const float* scale, const float* grad_w_hat, int64_t d_out, int64_t d_in,
               float grad_scale, float* grad_w, float* grad_scale_out, float* w_hat, void* workspace,
               size_t workspace_bytes, hipStream_t stream);
int w4a16_gemm_pc(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* scale_f16,
                  int64_t d_out, int64_t d_in, void* y, int y_dtype, int w_mode, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------- joint objective across the groups
 * [card] "Quantization Configuration" read over a whole output row: ||(w - w_hat) X||^2 =
 * e^T H e with the full H couples the groups of the row through the off-diagonal blocks of H
 * (quant_scale_search reads it per group, with the diagonal blocks only).
 *
 * quant_joint_objective -- obj[r] = e^T H e over row r, e = w - Delta_g * code(w, Delta_g) with the
 *   fp32 steps scale[r][g] (0, or fp32-normal and finite), full H (as in quant_scale_search_pc).
 *   obj fp64 [d_out] out.
 * quant_joint_refine -- coordinate descent over the groups of each row on that objective.  Start:
 *   idx [d_out][G] (in; e.g. quant_scale_search's choice; an index >= n_cand is read as
 *   n_cand - 1), steps Delta_k = candidate of the group
 *   as in quant_scale_search.  A sweep visits the groups in order; at group g every candidate is
 *   tried with the other groups held, and the first k with the smallest joint objective is kept
 *   (the current one is among them: the objective never rises).  Up to n_sweeps sweeps (>= 1),
 *   stopping after one that changes nothing.  Trials are scored exactly in fp64 as the change
 *   2 d^T u_g + d^T H_gg d of the objective (d = the group's error change, u = H e kept current
 *   through every accepted change; H must be symmetric, as quant_hessian writes it, since the
 *   change and the update of u read it by rows).  Outputs: idx (out: the result), scale fp32
 *   [d_out][G] out (its steps), obj_before / obj_after fp64 [d_out] or NULL, sweeps int32
 *   [d_out] or NULL (sweeps run per row).
 * joint_workspace_size -- bytes of the workspace both calls use to run all rows of up to 2048 at a
 *   time (u = H e for those rows in fp64 and partial objectives); any workspace of at least 64
 *   rows' share works, in more launches (W4Q_EINVAL below that, W4Q_EALIGN if misaligned).
 */
int joint_workspace_size(int64_t d_out, int64_t d_in, size_t* bytes);
int quant_joint_objective(const float* w, const float* scale, int64_t d_out, int64_t d_in,
                          const float* h, int64_t ldh, double* obj, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);
int quant_joint_refine(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
                       const float* alpha, int n_cand, uint8_t* idx, float* scale, int n_sweeps,
                       double* obj_before, double* obj_after, int32_t* sweeps, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------- GPTQ error feedback
 * quant_gptq -- GPTQ (the published algorithm of Frantar et al.; [blog] section 2 names it as the
 *   second-order reconstruction method the Hessian initialization starts from) on the group-32
 *   grid with fixed steps scale[r][g] (e.g. quant_scale_search's; static groups), columns in
 *   natural order.  H' = H with every dead column (H_ii == 0) given a unit diagonal and a zero
 *   weight, plus damp * mean(diag) on the diagonal.  Per row, column i is quantized from
 *   w'_i = w_i + (1 / R_ii) sum_{p < i} R_pi (w_p - w_hat_p),  H' = R R^T with R upper triangular,
 *   which is the least-squares update of the remaining weights given the columns already
 *   quantized (the published form's err / U_ii feedback through U = chol(H'^-1)^T = R^-1):
 *   w_hat_i = Delta * code(w'_i, Delta) with the exact nearest-code rule on the fp64 value.
 *   Everything in fp64 (fp64 matrix cores for the Cholesky update and the feedback sums).
 *   w      fp32 [d_out][d_in], 16-B aligned;  h fp32 [d_in][ldh] (all entries read; 16-B aligned,
 *          ldh >= d_in, ldh % 4 == 0);  scale fp32 [d_out][G] (0 or fp32-normal, finite);
 *   damp   >= 0 and finite (0.01 is the published default);
 *   w_hat  fp32 [d_out][d_in] out: Delta * q (exact for steps on the fp16 grid; quant_pack(w_hat,
 *          scale) then gives exactly these codes);
 *   info   int32 device scalar, or NULL: set to 1 if a Cholesky pivot of H' is not positive
 *          (w_hat is then unspecified); never cleared by the call.
 *   workspace: gptq_workspace_size bytes, 256-B aligned (W4Q_EINVAL if smaller or NULL,
 *          W4Q_EALIGN if misaligned): H' factor (d_in rounded up to 64, squared, fp64) and the
 *          rows' fp64 quantization errors.
 */
int gptq_workspace_size(int64_t d_out, int64_t d_in, size_t* bytes);
int quant_gptq(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
               const float* scale, float damp, float* w_hat, int32_t* info, void* workspace,
               size_t workspace_bytes, hipStream_t stream);

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
 *   w4q_probe_mfma_f64   likewise for 8 independent 16x16x4 fp64 products per wavefront, four
 *                        wavefronts per SIMD; sink is 8-B aligned device memory of
 *                        W4Q_PROBE_SINK_WORDS / 2 doubles (W4Q_EALIGN if misaligned).
 * Each enqueues one kernel on `stream` and returns W4Q_EINVAL for bad arguments.
 */
#define W4Q_PROBE_SINK_WORDS 65536
int w4q_probe_read(const void* buf, int64_t bytes, int nontemporal, uint32_t* sink, hipStream_t stream);
int w4q_probe_mfma_bf16(float* sink, int64_t iters, double* flop, hipStream_t stream);
int w4q_probe_mfma_f64(double* sink, int64_t iters, double* flop, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* W4A16Q_H */

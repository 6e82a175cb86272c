/*
 * oracle.c -- plain, slow, CPU reference of the W4A16 group-wise quantization core.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this code: only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no source
 * with the HIP library (own fp16 helpers, own code rule, own loops) and follows the pages
 * directly:
 *   [card]  model card "Opt.Gear-1B-qat-int4-per-channel-unquantized":
 *           "Quantization Configuration" (symmetric, zero-point 0; the objective
 *           Delta* = argmin_Delta ||W X - Q_Delta(W) X||_F^2), "QAT Highlights".
 *   [blog]  "Opt.Gear-QAT: Preserving On-Device Performance with QAT":
 *           "Quantization parameters of Opt.Gear-1B" (group 32, symmetric),
 *           "2. Hessian-based scale initialize", "3. LSQ-based QAT", "Conclusion".
 * Floating point is fp64 wherever the pages leave the precision open.  OpenMP is used only
 * across independent rows / groups / entries; every individual sum runs in plain index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GROUP 32
#define QMIN (-8)
#define QMAX 7

int orc_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------- 16-bit float formats */

/* IEEE 754 binary16 from fp32, round to nearest, ties to even; overflow -> infinity. */
uint16_t orc_f32_to_f16(float f) {
  uint32_t bits;
  memcpy(&bits, &f, 4);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if ((bits & 0x7F800000u) == 0x7F800000u) /* inf or nan */
    return (uint16_t)(sign | 0x7C00u | ((bits & 0x007FFFFFu) ? 0x0200u : 0u));
  double v = fabs((double)f);
  if (v == 0.0) return sign;
  int e;
  frexp(v, &e);
  int ex = e - 1;            /* v in [2^ex, 2^(ex+1)) */
  if (ex < -14) ex = -14;    /* subnormals share the quantum 2^-24 */
  double quantum = ldexp(1.0, ex - 10);
  double r = v / quantum;    /* exact (power-of-two scaling) */
  double n = floor(r);
  double frac = r - n;       /* exact */
  if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;
  double out = n * quantum;
  if (out >= 65536.0) return (uint16_t)(sign | 0x7C00u);
  if (out < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)(out / ldexp(1.0, -24)));
  frexp(out, &e);
  int E = e - 1;
  double mant = out / ldexp(1.0, E) - 1.0; /* in [0, 1), a multiple of 2^-10 */
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(mant * 1024.0));
}

/* binary16 bits -> value. */
double orc_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1F;
  int man = h & 0x3FF;
  double v;
  if (ex == 0) v = ldexp((double)man, -24);
  else if (ex == 31) v = man ? NAN : INFINITY;
  else v = ldexp(1.0 + man / 1024.0, ex - 15);
  return sign ? -v : v;
}

/* bfloat16 bits -> value (the upper half of an fp32 pattern). */
double orc_bf16_to_f64(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* ------------------------------------------------------------------- the INT4 grid */

/*
 * The symmetric INT4 grid with zero-point 0 ([card] configuration table; [blog]
 * "Quantization parameters") has the points c * D for c in [-8, 7].  The code of w is the
 * nearest grid point for the exact real quotient w / D, ties to the even code; this is
 * clamp(round_half_even(w / D), -8, 7).  It is found by walking the midpoints
 * (c + 1/2) * D, which are exact in fp64 (D has at most 24 significant bits, c + 1/2 at
 * most 5).  D == 0 gives code 0.
 */
int orc_code(double w, double d) {
  if (d == 0.0) return 0;
  int q = QMIN;
  for (int c = QMIN; c < QMAX; ++c) {
    double mid = (c + 0.5) * d;
    if (w > mid) {
      q = c + 1;
    } else if (w == mid) { /* equidistant from c and c + 1: take the even one */
      q = (c % 2 == 0) ? c : c + 1;
      break;
    } else {
      break;
    }
  }
  return q;
}

/*
 * Candidate scale k of a group: the max-based scale amax / 7 ([blog] section 2 names it as
 * the plain RTN choice) stretched by alpha_k, evaluated in fp32 in this order and then put
 * on the fp16 grid the deployed scales live on ([card] "QAT Highlights": one grid for
 * initialisation, QAT and export).
 */
float orc_candidate(float amax, float alpha) {
  float t = alpha * amax;
  float u = t / 7.0f;
  return (float)orc_f16_to_f64(orc_f32_to_f16(u));
}

/* -------------------------------------------------------------- calibration Hessian */

/* H = X^T X in fp64 for X [n][d] bf16 ([blog] section 2, second-order view).  Full matrix. */
void orc_hessian(const uint16_t* x, int64_t n, int64_t d, double* h) {
  /* column-major fp64 copy so each entry is one contiguous dot product over tokens */
  double* xt = (double*)malloc(sizeof(double) * (size_t)n * (size_t)d);
  for (int64_t t = 0; t < n; ++t)
    for (int64_t i = 0; i < d; ++i) xt[i * n + t] = orc_bf16_to_f64(x[t * d + i]);
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t i = 0; i < d; ++i) {
    for (int64_t j = i; j < d; ++j) {
      double s = 0.0;
      for (int64_t t = 0; t < n; ++t) s += xt[i * n + t] * xt[j * n + t];
      h[i * d + j] = s;
      h[j * d + i] = s;
    }
  }
  free(xt);
}

/* Selected entries H[ij[2c]][ij[2c+1]] of X^T X in fp64. */
void orc_hessian_entries(const uint16_t* x, int64_t n, int64_t d, const int64_t* ij, int64_t cnt,
                         double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < cnt; ++c) {
    int64_t i = ij[2 * c], j = ij[2 * c + 1];
    double s = 0.0;
    for (int64_t t = 0; t < n; ++t) s += orc_bf16_to_f64(x[t * d + i]) * orc_bf16_to_f64(x[t * d + j]);
    out[c] = s;
  }
}

/* ------------------------------------------------------------------ scale search */

/*
 * One group of n consecutive weights ([card] "Quantization Configuration" objective, read per
 * group with the group's diagonal block of H): returns the chosen index, its scale and
 * objective, and optionally every candidate's objective.  hg points at the block's first entry
 * with row stride ldh.  n = 32 is the [blog] group; n = d_in is one scale per output row (the
 * [card] per-channel checkpoint), where the block is the whole H.
 */
static void search_span(const float* wg, int64_t n, const float* hg, int64_t ldh,
                        const float* alpha, int K, float* scale, uint8_t* idx, double* obj,
                        double* obj_all) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i)
    if (fabsf(wg[i]) > amax) amax = fabsf(wg[i]);
  double* e = (double*)malloc((size_t)n * sizeof(double));
  double best = INFINITY;
  int kbest = 0;
  float dbest = 0.0f;
  for (int k = 0; k < K; ++k) {
    float dk = orc_candidate(amax, alpha[k]);
    double d = (double)dk;
    for (int64_t i = 0; i < n; ++i) e[i] = (double)wg[i] - d * (double)orc_code((double)wg[i], d);
    double o = 0.0;
    for (int64_t i = 0; i < n; ++i)
      for (int64_t j = 0; j < n; ++j) o += e[i] * (double)hg[i * ldh + j] * e[j];
    if (obj_all) obj_all[k] = o;
    if (o < best) { /* strict: the first minimum wins */
      best = o;
      kbest = k;
      dbest = dk;
    }
  }
  free(e);
  *scale = dbest;
  *idx = (uint8_t)kbest;
  *obj = best;
}

static void search_group(const float* wg, const float* hg, int64_t ldh, const float* alpha, int K,
                         float* scale, uint8_t* idx, double* obj, double* obj_all) {
  search_span(wg, GROUP, hg, ldh, alpha, K, scale, idx, obj, obj_all);
}

/* Every group of W [d_out][d_in].  obj [d_out][G]; obj_all [d_out][G][K] or NULL. */
void orc_scale_search(const float* w, int64_t d_out, int64_t d_in, const float* h, int64_t ldh,
                      const float* alpha, int K, float* scale, uint8_t* idx, double* obj,
                      double* obj_all) {
  int64_t G = d_in / GROUP;
#pragma omp parallel for schedule(static)
  for (int64_t rg = 0; rg < d_out * G; ++rg) {
    int64_t r = rg / G, g = rg % G;
    search_group(w + r * d_in + g * GROUP, h + g * GROUP * ldh + g * GROUP, ldh, alpha, K,
                 scale + rg, idx + rg, obj + rg, obj_all ? obj_all + rg * K : 0);
  }
}

/* Selected groups (rows[c], groups[c]) of W with row length d_in; outputs indexed by c. */
void orc_scale_search_groups(const float* w, int64_t d_in, const float* h, int64_t ldh,
                             const float* alpha, int K, const int64_t* rows,
                             const int64_t* groups, int64_t cnt, float* scale, uint8_t* idx,
                             double* obj, double* obj_all) {
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < cnt; ++c) {
    int64_t r = rows[c], g = groups[c];
    search_group(w + r * d_in + g * GROUP, h + g * GROUP * ldh + g * GROUP, ldh, alpha, K,
                 scale + c, idx + c, obj + c, obj_all ? obj_all + c * K : 0);
  }
}

/* Per-channel search on selected rows: the whole row is one group and H is used in full.
 * Outputs indexed by c: scale, idx, obj [cnt]; obj_all [cnt][K] or NULL. */
void orc_scale_search_pc(const float* w, int64_t d_in, const float* h, int64_t ldh,
                         const float* alpha, int K, const int64_t* rows, int64_t cnt, float* scale,
                         uint8_t* idx, double* obj, double* obj_all) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t c = 0; c < cnt; ++c)
    search_span(w + rows[c] * d_in, d_in, h, ldh, alpha, K, scale + c, idx + c, obj + c,
                obj_all ? obj_all + c * K : 0);
}

/* ------------------------------------------------------------------------- export */

/*
 * Export on the deployment grid ([card] "QAT Highlights"/"Quickstart", [blog]
 * "Conclusion"): fp16 scale, codes on that scale, two's-complement nibbles, low nibble
 * first.
 */
void orc_pack_g(const float* w, const float* scale, int64_t d_out, int64_t d_in, int64_t gsz,
                uint8_t* packed, uint16_t* s16) {
  int64_t G = d_in / gsz;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < d_out; ++r) {
    for (int64_t g = 0; g < G; ++g) {
      uint16_t hs = orc_f32_to_f16(scale[r * G + g]);
      s16[r * G + g] = hs;
      double d = orc_f16_to_f64(hs);
      for (int64_t i = 0; i < gsz; i += 2) {
        int64_t k = g * gsz + i;
        int q0 = orc_code((double)w[r * d_in + k], d);
        int q1 = orc_code((double)w[r * d_in + k + 1], d);
        packed[r * (d_in / 2) + k / 2] = (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
      }
    }
  }
}

void orc_pack(const float* w, const float* scale, int64_t d_out, int64_t d_in, uint8_t* packed,
              uint16_t* s16) {
  orc_pack_g(w, scale, d_out, d_in, GROUP, packed, s16);
}

/* Decode one packed code (two's-complement nibble). */
int orc_unpack(const uint8_t* packed_row, int64_t k) {
  int nib = (packed_row[k / 2] >> (4 * (k % 2))) & 0xF;
  return nib >= 8 ? nib - 16 : nib;
}

/* ----------------------------------------------------------------------------- LSQ */

/* [blog] section 3 forward: w_hat = Delta * code(w, Delta) with the fp32 learnable Delta. */
void orc_lsq_fwd_g(const float* w, const float* scale, int64_t d_out, int64_t d_in, int64_t gsz,
                   float* w_hat) {
  int64_t G = d_in / gsz;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < d_out; ++r)
    for (int64_t k = 0; k < d_in; ++k) {
      double d = (double)scale[r * G + k / gsz];
      int q = orc_code((double)w[r * d_in + k], d);
      w_hat[r * d_in + k] = (float)(d * q); /* exact product, one rounding to fp32 */
    }
}

void orc_lsq_fwd(const float* w, const float* scale, int64_t d_out, int64_t d_in, float* w_hat) {
  orc_lsq_fwd_g(w, scale, d_out, d_in, GROUP, w_hat);
}

/*
 * [blog] section 3 backward: straight-through estimator for round inside the clamp range
 * (grad_w = G there, 0 outside), and the LSQ step-size gradient
 * d w_hat / d Delta = q - w/Delta inside, the clamp level outside, summed over the group and
 * multiplied by the normalisation factor gs.  Range test -8*D <= w <= 7*D is exact in fp64.
 */
void orc_lsq_bwd_g(const float* w, const float* scale, const float* gup, int64_t d_out,
                   int64_t d_in, int64_t gsz, double gs, float* grad_w, double* grad_scale,
                   float* w_hat) {
  int64_t G = d_in / gsz;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < d_out; ++r)
    for (int64_t g = 0; g < G; ++g) {
      double d = (double)scale[r * G + g];
      double acc = 0.0;
      for (int64_t i = 0; i < gsz; ++i) {
        int64_t k = r * d_in + g * gsz + i;
        double wv = (double)w[k];
        int q = orc_code(wv, d);
        int in_range = (wv >= QMIN * d) && (wv <= QMAX * d);
        grad_w[k] = in_range ? gup[k] : 0.0f;
        double f = in_range ? (double)q - wv / d : (double)q;
        acc += (double)gup[k] * f;
        if (w_hat) w_hat[k] = (float)(d * q);
      }
      grad_scale[r * G + g] = gs * acc;
    }
}

void orc_lsq_bwd(const float* w, const float* scale, const float* gup, int64_t d_out, int64_t d_in,
                 double gs, float* grad_w, double* grad_scale, float* w_hat) {
  orc_lsq_bwd_g(w, scale, gup, d_out, d_in, GROUP, gs, grad_w, grad_scale, w_hat);
}

/* ------------------------------------------------------------------------ W4A16 GEMM */

/*
 * Deployment product ([card] intro: INT4 weights, 16-bit activations):
 * y[m][c] = sum_k x[m][k] * s16[n][k/32] * q[n][k] for n = cols[c], in fp64; yabs receives
 * sum_k |x[m][k] * w_hat[n][k]| (the scale of the rounding-error bound).
 */
/* The nearest bfloat16 value (8 significant bits) to a finite v, ties to the even
 * significand.  v is a product s16 * q here: exact in fp64, far inside the bf16 range. */
double orc_round_bf16(double v) {
  if (v == 0.0) return v;
  double a = fabs(v);
  int e;
  frexp(a, &e);
  double quantum = ldexp(1.0, e - 1 - 7); /* a in [2^(e-1), 2^e): 7 fraction bits */
  double r = a / quantum;                 /* exact */
  double n = floor(r);
  double frac = r - n;
  if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;
  double out = n * quantum;
  return v < 0 ? -out : out;
}

/* y = x W_hat^T on the chosen output columns.  Two readings of the dequantized weight:
 *   dq = 0: w_hat = s16 * q exactly ([card] W4A16 deployment with the [blog] group grid);
 *   dq = 1: w_hat = bf16_RNE(s16 * q), the weight as a bf16 operand of the matrix product
 *           (dequantization to the 16-bit activation format before the product). */
void orc_gemm_cols_g(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                     int64_t d_in, int64_t gsz, const int64_t* cols, int64_t ncols, int dq, double* y,
                     double* yabs) {
  int64_t G = d_in / gsz;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < ncols; ++c) {
    int64_t n = cols[c];
    const uint8_t* prow = packed + n * (d_in / 2);
    for (int64_t mi = 0; mi < m; ++mi) {
      double s = 0.0, sa = 0.0;
      for (int64_t k = 0; k < d_in; ++k) {
        double wh = orc_f16_to_f64(s16[n * G + k / gsz]) * (double)orc_unpack(prow, k);
        if (dq) wh = orc_round_bf16(wh);
        double p = orc_bf16_to_f64(x[mi * d_in + k]) * wh;
        s += p;
        sa += fabs(p);
      }
      y[mi * ncols + c] = s;
      if (yabs) yabs[mi * ncols + c] = sa;
    }
  }
}

void orc_gemm_cols_mode(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                        int64_t d_in, const int64_t* cols, int64_t ncols, int dq, double* y, double* yabs) {
  orc_gemm_cols_g(x, m, packed, s16, d_in, GROUP, cols, ncols, dq, y, yabs);
}

/* ------------------------------------------------------------ fused QAT update (Adam) */

/*
 * One optimisation step of QAT with LSQ ([blog] section 3: weights and step sizes are learned
 * jointly; [card] "QAT Highlights": the forward emulates the deployment grid), for one linear:
 * the LSQ / straight-through gradients of orc_lsq_bwd, then Adam on both (decoupled weight decay
 * on W only; the step is kept at or above scale_min), and optionally the fake-quantised updated
 * weights for the next forward.  hp = {lr_w, lr_s, beta1, beta2, eps, weight_decay, c1, c2,
 * scale_min} with c1 = 1 - beta1^t, c2 = 1 - beta2^t.  Per element, in fp64:
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2
 *   w = w - lr_w ((m / c1) / (sqrt(v / c2) + eps) + weight_decay w)
 *   D = max(D - lr_s (m_s / c1) / (sqrt(v_s / c2) + eps), scale_min)
 * ext_ds (nullable) replaces the computed step-size gradients (to check the update alone on
 * given gradients).  Outputs are rounded to fp32 once.
 */
void orc_lsq_adam_step(const float* w, const float* scale, const float* gup, int64_t d_out,
                       int64_t d_in, double gs, const float* m_w, const float* v_w,
                       const float* m_s, const float* v_s, const double* hp, const double* ext_ds,
                       float* w_out, float* scale_out, float* m_w_out, float* v_w_out,
                       float* m_s_out, float* v_s_out, double* ds_out, float* w_hat_next) {
  const double lr_w = hp[0], lr_s = hp[1], b1 = hp[2], b2 = hp[3], eps = hp[4], wd = hp[5];
  const double c1 = hp[6], c2 = hp[7], smin = hp[8];
  int64_t G = d_in / GROUP;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < d_out; ++r)
    for (int64_t g = 0; g < G; ++g) {
      int64_t gi = r * G + g;
      double d = (double)scale[gi];
      double acc = 0.0;
      for (int64_t i = 0; i < GROUP; ++i) {
        int64_t k = r * d_in + g * GROUP + i;
        double wv = (double)w[k];
        int q = orc_code(wv, d);
        int in_range = (wv >= QMIN * d) && (wv <= QMAX * d);
        double gw = in_range ? (double)gup[k] : 0.0;
        double f = in_range ? (double)q - wv / d : (double)q;
        acc += (double)gup[k] * f;
        double m = b1 * (double)m_w[k] + (1.0 - b1) * gw;
        double v = b2 * (double)v_w[k] + (1.0 - b2) * gw * gw;
        double wn = wv - lr_w * ((m / c1) / (sqrt(v / c2) + eps) + wd * wv);
        m_w_out[k] = (float)m;
        v_w_out[k] = (float)v;
        w_out[k] = (float)wn;
      }
      double ds = ext_ds ? ext_ds[gi] : gs * acc;
      if (ds_out) ds_out[gi] = ds;
      double ms = b1 * (double)m_s[gi] + (1.0 - b1) * ds;
      double vs = b2 * (double)v_s[gi] + (1.0 - b2) * ds * ds;
      double dn = d - lr_s * (ms / c1) / (sqrt(vs / c2) + eps);
      if (dn < smin) dn = smin;
      m_s_out[gi] = (float)ms;
      v_s_out[gi] = (float)vs;
      scale_out[gi] = (float)dn;
      if (w_hat_next) {
        double dd = (double)scale_out[gi]; /* the fp32 step the next forward uses */
        for (int64_t i = 0; i < GROUP; ++i) {
          int64_t k = r * d_in + g * GROUP + i;
          int q = orc_code((double)w_out[k], dd);
          w_hat_next[k] = (float)(dd * q);
        }
      }
    }
}

/* ---------------------------------------------------- joint objective across groups */

/* e = w - Delta_g * code(w, Delta_g) for one row, Delta_g = step[g] (fp32 as given), exact. */
static void row_error(const float* wr, const double* step, int64_t d_in, double* e) {
  for (int64_t k = 0; k < d_in; ++k) {
    double d = step[k / GROUP];
    e[k] = (double)wr[k] - d * (double)orc_code((double)wr[k], d);
  }
}

/* e^T H e over the whole row, full H, plain index order. */
static double row_form(const double* e, int64_t d_in, const float* h, int64_t ldh) {
  double o = 0.0;
  for (int64_t i = 0; i < d_in; ++i)
    for (int64_t j = 0; j < d_in; ++j) o += e[i] * (double)h[i * ldh + j] * e[j];
  return o;
}

/*
 * The [card] "Quantization Configuration" objective read literally for one output row:
 * ||(w - w_hat) X||^2 = e^T H e with the full H, which couples the groups of the row through the
 * off-diagonal blocks of H.  w_hat is the group-32 grid on the given fp32 steps scale[r][g].
 * Selected rows; obj [cnt].
 */
void orc_joint_objective(const float* w, const float* scale, int64_t d_in, const float* h,
                         int64_t ldh, const int64_t* rows, int64_t cnt, double* obj) {
  int64_t G = d_in / GROUP;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t c = 0; c < cnt; ++c) {
    int64_t r = rows[c];
    double* step = (double*)malloc((size_t)G * sizeof(double));
    double* e = (double*)malloc((size_t)d_in * sizeof(double));
    for (int64_t g = 0; g < G; ++g) step[g] = (double)scale[r * G + g];
    row_error(w + r * d_in, step, d_in, e);
    obj[c] = row_form(e, d_in, h, ldh);
    free(step);
    free(e);
  }
}

/*
 * Coordinate descent over the groups of a row on that joint objective.  The start is one
 * candidate index per group (idx, e.g. the per-group choice).  A sweep visits the groups in
 * order; at group g each candidate step Delta_k = candidate(amax_g, alpha_k) is tried with the
 * other groups held, its joint objective evaluated in full, and the first k with the smallest
 * objective is kept.  The current index is one of the candidates, so the objective never rises.
 * Sweeps repeat up to n_sweeps times and stop after one that changes nothing.
 * Outputs per selected row c: idx [cnt][G] (in: start, out: result), scale [cnt][G] (the steps
 * of the result), obj [cnt] (its joint objective), sweeps [cnt] (sweeps run), and margin [cnt]:
 * over all decisions, the smallest (o_k - o_kept) / o_kept among candidates whose step differs
 * from the kept one (+inf if none); a small margin marks a near-tie.
 */
void orc_joint_refine(const float* w, int64_t d_in, const float* h, int64_t ldh,
                      const float* alpha, int K, const int64_t* rows, int64_t cnt, int n_sweeps,
                      uint8_t* idx, float* scale, double* obj, double* margin, int* sweeps) {
  int64_t G = d_in / GROUP;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t c = 0; c < cnt; ++c) {
    const float* wr = w + rows[c] * d_in;
    uint8_t* ir = idx + c * G;
    float* cand = (float*)malloc((size_t)(G * K) * sizeof(float));
    double* step = (double*)malloc((size_t)G * sizeof(double));
    double* e = (double*)malloc((size_t)d_in * sizeof(double));
    double* o = (double*)malloc((size_t)K * sizeof(double));
    for (int64_t g = 0; g < G; ++g) {
      float amax = 0.0f;
      for (int i = 0; i < GROUP; ++i)
        if (fabsf(wr[g * GROUP + i]) > amax) amax = fabsf(wr[g * GROUP + i]);
      for (int k = 0; k < K; ++k) cand[g * K + k] = orc_candidate(amax, alpha[k]);
      step[g] = (double)cand[g * K + ir[g]];
    }
    double mg = INFINITY;
    int s = 0;
    while (s < n_sweeps) {
      ++s;
      int changed = 0;
      for (int64_t g = 0; g < G; ++g) {
        int kb = 0;
        for (int k = 0; k < K; ++k) {
          step[g] = (double)cand[g * K + k];
          row_error(wr, step, d_in, e);
          o[k] = row_form(e, d_in, h, ldh);
          if (o[k] < o[kb]) kb = k; /* strict: the first minimum wins */
        }
        for (int k = 0; k < K; ++k)
          if (cand[g * K + k] != cand[g * K + kb] && o[kb] > 0.0) {
            double gap = (o[k] - o[kb]) / o[kb];
            if (gap < mg) mg = gap;
          }
        if (kb != ir[g]) {
          ir[g] = (uint8_t)kb;
          changed = 1;
        }
        step[g] = (double)cand[g * K + kb];
      }
      if (!changed) break;
    }
    for (int64_t g = 0; g < G; ++g) scale[c * G + g] = (float)step[g];
    row_error(wr, step, d_in, e);
    obj[c] = row_form(e, d_in, h, ldh);
    margin[c] = mg;
    sweeps[c] = s;
    free(cand);
    free(step);
    free(e);
    free(o);
  }
}

/* ------------------------------------------------ GPTQ-style error feedback (prior art) */

/* In-place Cholesky a = L L^T of an n x n symmetric matrix (row-major, lower triangle used);
 * L left in the lower triangle.  Returns 0, or 1 if a pivot is not positive. */
static int chol_lower(double* a, int64_t n) {
  for (int64_t j = 0; j < n; ++j) {
    double s = a[j * n + j];
    for (int64_t p = 0; p < j; ++p) s -= a[j * n + p] * a[j * n + p];
    if (!(s > 0.0)) return 1;
    double d = sqrt(s);
    a[j * n + j] = d;
#pragma omp parallel for schedule(static)
    for (int64_t i = j + 1; i < n; ++i) {
      double t = a[i * n + j];
      for (int64_t p = 0; p < j; ++p) t -= a[i * n + p] * a[j * n + p];
      a[i * n + j] = t / d;
    }
  }
  return 0;
}

/*
 * GPTQ (Frantar et al., "GPTQ: Accurate Post-Training Quantization for Generative Pre-trained
 * Transformers", the published algorithm; [blog] section 2 names it as the second-order output
 * reconstruction method the Hessian initialization starts from) on the group-32 grid with the
 * caller's fixed steps scale[r][g] (static groups), columns in natural order:
 *   dead columns (H_ii == 0): H_ii = 1 and w_i = 0;  H' = H + damp * mean(diag H) I;
 *   U = the upper Cholesky factor of H'^-1 (H'^-1 = U^T U);
 *   per row, for i = 0 .. d_in-1:  q = code(w_i, Delta_g(i));  w_hat_i = Delta q;
 *     err = (w_i - w_hat_i) / U_ii;  w_j -= err * U_ij for every j > i.
 * Selected rows; w_hat [cnt][d_in] (fp32 of the exact product), w_upd [cnt][d_in] or NULL (the
 * updated weight each column was quantized from), margin [cnt] or NULL: the smallest distance,
 * in steps, of an updated weight w_i / Delta from a decision midpoint c + 1/2 (c = -8 .. 6).
 * Returns 0, or 1 if H' is not positive definite.
 */
int orc_gptq(const float* w, int64_t d_in, const float* h, int64_t ldh, const float* scale,
             double damp, const int64_t* rows, int64_t cnt, float* w_hat, double* w_upd,
             double* margin) {
  int64_t n = d_in, G = d_in / GROUP;
  double* hd = (double*)malloc((size_t)(n * n) * sizeof(double));
  double* inv = (double*)malloc((size_t)(n * n) * sizeof(double));
  unsigned char* dead = (unsigned char*)malloc((size_t)n);
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < n; ++j) hd[i * n + j] = (double)h[i * ldh + j];
  double mean = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    dead[i] = hd[i * n + i] == 0.0;
    if (dead[i]) hd[i * n + i] = 1.0;
    mean += hd[i * n + i];
  }
  mean /= (double)n;
  for (int64_t i = 0; i < n; ++i) hd[i * n + i] += damp * mean;
  /* H'^-1 from H' = L L^T: column c of the inverse solves L L^T x = e_c */
  int bad = chol_lower(hd, n);
  if (!bad) {
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t c = 0; c < n; ++c) {
      double* x = (double*)malloc((size_t)n * sizeof(double));
      for (int64_t i = 0; i < n; ++i) { /* L y = e_c */
        double t = (i == c) ? 1.0 : 0.0;
        for (int64_t p = 0; p < i; ++p) t -= hd[i * n + p] * x[p];
        x[i] = t / hd[i * n + i];
      }
      for (int64_t i = n - 1; i >= 0; --i) { /* L^T x = y */
        double t = x[i];
        for (int64_t p = i + 1; p < n; ++p) t -= hd[p * n + i] * x[p];
        x[i] = t / hd[i * n + i];
      }
      for (int64_t i = 0; i < n; ++i) inv[i * n + c] = x[i];
      free(x);
    }
    bad = chol_lower(inv, n); /* inv = L2 L2^T, U = L2^T: U_ij = inv[j][i] for j >= i */
  }
  if (!bad) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < cnt; ++c) {
      int64_t r = rows[c];
      double* wr = (double*)malloc((size_t)n * sizeof(double));
      double mg = INFINITY;
      for (int64_t i = 0; i < n; ++i) wr[i] = dead[i] ? 0.0 : (double)w[r * d_in + i];
      for (int64_t i = 0; i < n; ++i) {
        double d = (double)scale[r * G + i / GROUP];
        int q = orc_code(wr[i], d);
        double wh = d * (double)q;
        if (d > 0.0)
          for (int k = QMIN; k < QMAX; ++k) {
            double dist = fabs(wr[i] / d - ((double)k + 0.5));
            if (dist < mg) mg = dist;
          }
        if (w_upd) w_upd[c * n + i] = wr[i];
        w_hat[c * n + i] = (float)wh;
        double err = (wr[i] - wh) / inv[i * n + i];
        for (int64_t j = i + 1; j < n; ++j) wr[j] -= err * inv[j * n + i];
      }
      if (margin) margin[c] = mg;
      free(wr);
    }
  }
  free(hd);
  free(inv);
  free(dead);
  return bad;
}

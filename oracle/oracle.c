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
 * One group ([card] "Quantization Configuration" objective, read per group of 32 with the
 * group's diagonal block of H): returns the chosen index, its scale and objective, and
 * optionally every candidate's objective.  hg points at H[32g][32g] with row stride ldh.
 */
static void search_group(const float* wg, const float* hg, int64_t ldh, const float* alpha, int K,
                         float* scale, uint8_t* idx, double* obj, double* obj_all) {
  float amax = 0.0f;
  for (int i = 0; i < GROUP; ++i)
    if (fabsf(wg[i]) > amax) amax = fabsf(wg[i]);
  double best = INFINITY;
  int kbest = 0;
  float dbest = 0.0f;
  for (int k = 0; k < K; ++k) {
    float dk = orc_candidate(amax, alpha[k]);
    double d = (double)dk;
    double e[GROUP];
    for (int i = 0; i < GROUP; ++i) e[i] = (double)wg[i] - d * (double)orc_code((double)wg[i], d);
    double o = 0.0;
    for (int i = 0; i < GROUP; ++i)
      for (int j = 0; j < GROUP; ++j) o += e[i] * (double)hg[i * ldh + j] * e[j];
    if (obj_all) obj_all[k] = o;
    if (o < best) { /* strict: the first minimum wins */
      best = o;
      kbest = k;
      dbest = dk;
    }
  }
  *scale = dbest;
  *idx = (uint8_t)kbest;
  *obj = best;
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

/* ------------------------------------------------------------------------- export */

/*
 * Export on the deployment grid ([card] "QAT Highlights"/"Quickstart", [blog]
 * "Conclusion"): fp16 scale, codes on that scale, two's-complement nibbles, low nibble
 * first.
 */
void orc_pack(const float* w, const float* scale, int64_t d_out, int64_t d_in, uint8_t* packed,
              uint16_t* s16) {
  int64_t G = d_in / GROUP;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < d_out; ++r) {
    for (int64_t g = 0; g < G; ++g) {
      uint16_t hs = orc_f32_to_f16(scale[r * G + g]);
      s16[r * G + g] = hs;
      double d = orc_f16_to_f64(hs);
      for (int64_t i = 0; i < GROUP; i += 2) {
        int64_t k = g * GROUP + i;
        int q0 = orc_code((double)w[r * d_in + k], d);
        int q1 = orc_code((double)w[r * d_in + k + 1], d);
        packed[r * (d_in / 2) + k / 2] = (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
      }
    }
  }
}

/* Decode one packed code (two's-complement nibble). */
int orc_unpack(const uint8_t* packed_row, int64_t k) {
  int nib = (packed_row[k / 2] >> (4 * (k % 2))) & 0xF;
  return nib >= 8 ? nib - 16 : nib;
}

/* ----------------------------------------------------------------------------- LSQ */

/* [blog] section 3 forward: w_hat = Delta * code(w, Delta) with the fp32 learnable Delta. */
void orc_lsq_fwd(const float* w, const float* scale, int64_t d_out, int64_t d_in, float* w_hat) {
  int64_t G = d_in / GROUP;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < d_out; ++r)
    for (int64_t k = 0; k < d_in; ++k) {
      double d = (double)scale[r * G + k / GROUP];
      int q = orc_code((double)w[r * d_in + k], d);
      w_hat[r * d_in + k] = (float)(d * q); /* exact product, one rounding to fp32 */
    }
}

/*
 * [blog] section 3 backward: straight-through estimator for round inside the clamp range
 * (grad_w = G there, 0 outside), and the LSQ step-size gradient
 * d w_hat / d Delta = q - w/Delta inside, the clamp level outside, summed over the group and
 * multiplied by the normalisation factor gs.  Range test -8*D <= w <= 7*D is exact in fp64.
 */
void orc_lsq_bwd(const float* w, const float* scale, const float* gup, int64_t d_out, int64_t d_in,
                 double gs, float* grad_w, double* grad_scale, float* w_hat) {
  int64_t G = d_in / GROUP;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < d_out; ++r)
    for (int64_t g = 0; g < G; ++g) {
      double d = (double)scale[r * G + g];
      double acc = 0.0;
      for (int64_t i = 0; i < GROUP; ++i) {
        int64_t k = r * d_in + g * GROUP + i;
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
void orc_gemm_cols_mode(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                        int64_t d_in, const int64_t* cols, int64_t ncols, int dq, double* y, double* yabs) {
  int64_t G = d_in / GROUP;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < ncols; ++c) {
    int64_t n = cols[c];
    const uint8_t* prow = packed + n * (d_in / 2);
    for (int64_t mi = 0; mi < m; ++mi) {
      double s = 0.0, sa = 0.0;
      for (int64_t k = 0; k < d_in; ++k) {
        double wh = orc_f16_to_f64(s16[n * G + k / GROUP]) * (double)orc_unpack(prow, k);
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

void orc_gemm_cols(const uint16_t* x, int64_t m, const uint8_t* packed, const uint16_t* s16,
                   int64_t d_in, const int64_t* cols, int64_t ncols, double* y, double* yabs) {
  int64_t G = d_in / GROUP;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < ncols; ++c) {
    int64_t n = cols[c];
    const uint8_t* prow = packed + n * (d_in / 2);
    for (int64_t mi = 0; mi < m; ++mi) {
      double s = 0.0, sa = 0.0;
      for (int64_t k = 0; k < d_in; ++k) {
        double wh = orc_f16_to_f64(s16[n * G + k / GROUP]) * (double)orc_unpack(prow, k);
        double p = orc_bf16_to_f64(x[mi * d_in + k]) * wh;
        s += p;
        sa += fabs(p);
      }
      y[mi * ncols + c] = s;
      if (yabs) yabs[mi * ncols + c] = sa;
    }
  }
}

/*
 * oracle.c -- plain, slow, float64 CPU reference of one MoE layer of a
 * decode step.  TEST INFRASTRUCTURE ONLY: it is called by the tests, by the
 * package's smoke check and by the benchmark's CPU-baseline leg, never by
 * the library.  It shares no code with the HIP path (its own format parser,
 * its own dims struct) and takes host copies of the exact bytes the device
 * consumed.
 *
 * What it computes follows the Flash-MoE pages:
 *   "Flash-MoE: Running a 397B Parameter Model on a Laptop" (hysenlabs.com),
 *     section "How the SSD expert streaming pipeline works": per layer a
 *     router, a softmax and top-K routing (K=4 of 512 experts), the forward
 *     pass of the selected experts plus one shared expert, and a combine.
 *   "Flash-MoE: Running a 400 Billion Parameter Model on a MacBook"
 *     (mattcullerton.com), section "The Architecture": experts are 4-bit and
 *     dequantised inside the matrix-vector inner loop.
 * Readings where the pages are silent (each listed in the design notes):
 *   affine dequantisation w = s*q + z, unsigned codes, groups of 64 along the
 *   input dimension, bf16 s and z; softmax over all experts, then top-K, then
 *   renormalisation of the K kept probabilities; ties in the logits go to the
 *   lower expert index; SwiGLU h = silu(gate x) * (up x); the shared expert
 *   is added with weight 1.
 * Every sum is a plain sequential loop in double precision.  Independent
 * output rows (router logits, expert rows) may run on several threads
 * (OpenMP, or_set_threads); each row's sum is the same sequential loop, so
 * results do not depend on the thread count.
 *
 * Parity pins: see tests/test_oracle.py (hand-worked cases, closed forms,
 * identities, brute force).  No function here is "parity unpinned".
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t H, I, E, K, bits, group, has_shared;
} or_dims;

/* Threads used for independent output rows (1 = fully sequential). */
static int or_threads = 1;
void or_set_threads(int n) { or_threads = n < 1 ? 1 : n; }
int or_get_threads(void) { return or_threads; }

/* ---- bf16 ---------------------------------------------------------------- */

/* A bf16 value is the upper half of an IEEE fp32 bit pattern; widening is
 * exact. */
double or_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ---- blob format ----------------------------------------------------------
 * Sections in order gate codes, up codes, down codes, gate (s,z), up (s,z),
 * down (s,z); each starts 256-byte aligned.  Codes: `32/bits` per
 * little-endian 32-bit word, code c of a row at bit bits*(c mod 32/bits) of
 * word c/(32/bits).  (s,z) word [r][j]: low half s, high half z, bf16. */

static int64_t or_rows(const or_dims *d, int which) { return which == 2 ? d->H : d->I; }
static int64_t or_cols(const or_dims *d, int which) { return which == 2 ? d->I : d->H; }

int64_t or_section_offset(const or_dims *d, int sec) {
  int64_t off = 0;
  for (int s = 0; s < sec; ++s) {
    int which = s % 3;
    int64_t rows = or_rows(d, which), cols = or_cols(d, which);
    int64_t bytes = s < 3 ? rows * cols * d->bits / 8 : rows * (cols / d->group) * 4;
    off += bytes;
    off = (off + 255) / 256 * 256;
  }
  return off;
}

int64_t or_blob_bytes(const or_dims *d) { return or_section_offset(d, 6); }

static uint32_t or_word(const uint8_t *p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
         ((uint32_t)p[3] << 24);
}

/* One matrix of a blob: where its codes and (s,z) words are. */
typedef struct {
  const uint8_t *codes, *sb;
  int64_t rows, cols, words_per_row, groups;
  int32_t bits, group;
} or_mat;

or_mat or_matrix(const or_dims *d, const uint8_t *blob, int which) {
  or_mat m;
  m.rows = or_rows(d, which);
  m.cols = or_cols(d, which);
  m.bits = d->bits;
  m.group = d->group;
  m.words_per_row = m.cols / (32 / d->bits);
  m.groups = m.cols / d->group;
  m.codes = blob + or_section_offset(d, which);
  m.sb = blob + or_section_offset(d, 3 + which);
  return m;
}

/* Code q of element (r, c). */
static int32_t or_mat_code(const or_mat *m, int64_t r, int64_t c) {
  const int64_t cpw = 32 / m->bits;
  uint32_t w = or_word(m->codes + 4 * (r * m->words_per_row + c / cpw));
  return (int32_t)((w >> (m->bits * (c % cpw))) & ((1u << m->bits) - 1u));
}

/* Scale and bias of element (r, c). */
static void or_mat_sb(const or_mat *m, int64_t r, int64_t c, double *s, double *z) {
  uint32_t w = or_word(m->sb + 4 * (r * m->groups + c / m->group));
  *s = or_bf16((uint16_t)(w & 0xFFFFu));
  *z = or_bf16((uint16_t)(w >> 16));
}

/* Dequantised weight in double: s*q + z.  s*q is exact (a bf16 significand
 * of 8 bits times a code of at most 4 bits).  The sum with z is exact
 * whenever the two exponents are close enough for 53 bits to hold both,
 * which holds for any realistic scale and bias; TwoSum (Knuth) recovers the
 * rounding error of the sum and the program aborts if it is not zero, so the
 * returned double is always the exact real value. */
static double or_mat_dequant(const or_mat *m, int64_t r, int64_t c) {
  double s, z;
  or_mat_sb(m, r, c, &s, &z);
  double a = s * (double)or_mat_code(m, r, c);
  double sum = a + z;
  double bv = sum - a;
  double err = (a - (sum - bv)) + (z - bv);
  if (err != 0.0) {
    fprintf(stderr, "oracle: inexact dequant at r=%lld c=%lld\n", (long long)r, (long long)c);
    abort();
  }
  return sum;
}

/* Public element accessors (which: 0 gate, 1 up, 2 down). */
int32_t or_code(const or_dims *d, const uint8_t *blob, int which, int64_t r, int64_t c) {
  or_mat m = or_matrix(d, blob, which);
  return or_mat_code(&m, r, c);
}

void or_scale_bias(const or_dims *d, const uint8_t *blob, int which, int64_t r, int64_t c,
                   double *s, double *z) {
  or_mat m = or_matrix(d, blob, which);
  or_mat_sb(&m, r, c, s, z);
}

double or_dequant(const or_dims *d, const uint8_t *blob, int which, int64_t r, int64_t c) {
  or_mat m = or_matrix(d, blob, which);
  return or_mat_dequant(&m, r, c);
}

/* The same value rounded once to fp32 (round to nearest even). */
float or_dequant_f32(const or_dims *d, const uint8_t *blob, int which, int64_t r, int64_t c) {
  return (float)or_dequant(d, blob, which, r, c);
}

/* Whole matrix in double or fp32, row-major [rows][cols]. */
void or_dequant_matrix(const or_dims *d, const uint8_t *blob, int which, double *out) {
  or_mat m = or_matrix(d, blob, which);
  for (int64_t r = 0; r < m.rows; ++r)
    for (int64_t c = 0; c < m.cols; ++c) out[r * m.cols + c] = or_mat_dequant(&m, r, c);
}

void or_dequant_matrix_f32(const or_dims *d, const uint8_t *blob, int which, float *out) {
  or_mat m = or_matrix(d, blob, which);
  for (int64_t r = 0; r < m.rows; ++r)
    for (int64_t c = 0; c < m.cols; ++c)
      out[r * m.cols + c] = (float)or_mat_dequant(&m, r, c);
}

/* ---- routing -------------------------------------------------------------- */

/* Router logits of one token: l[e] = sum_c R[e][c] * x[c]. */
void or_router_logits(const or_dims *d, const uint16_t *router, const uint16_t *x,
                      double *logits) {
#pragma omp parallel for schedule(static) num_threads(or_threads)
  for (int64_t e = 0; e < d->E; ++e) {
    double acc = 0.0;
    for (int64_t c = 0; c < d->H; ++c)
      acc += or_bf16(router[e * d->H + c]) * or_bf16(x[c]);
    logits[e] = acc;
  }
}

/* Softmax over all experts, then the K largest logits (ties: lower index
 * first), then the K kept probabilities renormalised to sum to 1.
 * gap = smallest difference between consecutive logits among the ranks
 * 1..K+1 (ranks 1..K when E == K); it measures how far the selection and
 * its order are from a tie. */
void or_route_token(const or_dims *d, const double *logits, int32_t *ids, double *w,
                    double *gap) {
  const int E = d->E, K = d->K;
  /* softmax over all E */
  double m = logits[0];
  for (int e = 1; e < E; ++e)
    if (logits[e] > m) m = logits[e];
  double *p = (double *)malloc(sizeof(double) * E);
  int *order = (int *)malloc(sizeof(int) * E);
  double denom = 0.0;
  for (int e = 0; e < E; ++e) {
    p[e] = exp(logits[e] - m);
    denom += p[e];
  }
  for (int e = 0; e < E; ++e) p[e] /= denom;
  /* stable selection sort of the first K+1 ranks by (logit desc, index asc) */
  for (int e = 0; e < E; ++e) order[e] = e;
  const int ranks = K < E ? K + 1 : K;
  for (int r = 0; r < ranks; ++r) {
    int best = r;
    for (int j = r + 1; j < E; ++j) {
      int a = order[j], b = order[best];
      if (logits[a] > logits[b] || (logits[a] == logits[b] && a < b)) best = j;
    }
    int t = order[r];
    order[r] = order[best];
    order[best] = t;
  }
  double kept = 0.0;
  for (int k = 0; k < K; ++k) {
    ids[k] = order[k];
    kept += p[order[k]];
  }
  for (int k = 0; k < K; ++k) w[k] = p[order[k]] / kept;
  double g = INFINITY;
  for (int r = 0; r + 1 < ranks; ++r) {
    double diff = logits[order[r]] - logits[order[r + 1]];
    if (diff < g) g = diff;
  }
  *gap = g;
  free(p);
  free(order);
}

/* T tokens: logits [T][E] (may be NULL), ids [T][K], w [T][K], gap [T]. */
void or_route(const or_dims *d, const uint16_t *router, const uint16_t *x, int32_t T,
              int32_t *ids, double *w, double *logits, double *gap) {
  double *l = (double *)malloc(sizeof(double) * d->E);
  for (int32_t t = 0; t < T; ++t) {
    or_router_logits(d, router, x + (int64_t)t * d->H, l);
    if (logits) memcpy(logits + (int64_t)t * d->E, l, sizeof(double) * d->E);
    or_route_token(d, l, ids + (int64_t)t * d->K, w + (int64_t)t * d->K, gap + t);
  }
  free(l);
}

/* ---- expert MLP ----------------------------------------------------------- */

double or_silu(double v) { return v / (1.0 + exp(-v)); }

/* One expert on one token: g = Gate x, u = Up x, h = silu(g) * u,
 * y = Down h.  x has H doubles, y receives H doubles; h (I doubles, may be
 * NULL) receives the activations. */
void or_expert(const or_dims *d, const uint8_t *blob, const double *x, double *y, double *h_out) {
  const int64_t H = d->H, I = d->I;
  const or_mat gate = or_matrix(d, blob, 0), up = or_matrix(d, blob, 1),
               down = or_matrix(d, blob, 2);
  double *h = (double *)malloc(sizeof(double) * I);
#pragma omp parallel for schedule(static) num_threads(or_threads)
  for (int64_t r = 0; r < I; ++r) {
    double g = 0.0, u = 0.0;
    for (int64_t c = 0; c < H; ++c) g += or_mat_dequant(&gate, r, c) * x[c];
    for (int64_t c = 0; c < H; ++c) u += or_mat_dequant(&up, r, c) * x[c];
    h[r] = or_silu(g) * u;
  }
#pragma omp parallel for schedule(static) num_threads(or_threads)
  for (int64_t j = 0; j < H; ++j) {
    double acc = 0.0;
    for (int64_t r = 0; r < I; ++r) acc += or_mat_dequant(&down, j, r) * h[r];
    y[j] = acc;
  }
  if (h_out) memcpy(h_out, h, sizeof(double) * I);
  free(h);
}

/* ---- one layer ------------------------------------------------------------ */

/* Full layer for T tokens.  blobs[e] points at expert e's blob (host memory);
 * it may be NULL for experts that no token selects (the call aborts if a
 * selected expert is NULL).  shared may be NULL iff !has_shared.
 * Outputs: y [T][H]; ids [T][K]; w [T][K]; logits [T][E] (or NULL);
 * gap [T]. */
void or_layer(const or_dims *d, const uint16_t *router, const uint8_t *const *blobs,
              const uint8_t *shared, const uint16_t *x, int32_t T, double *y,
              int32_t *ids, double *w, double *logits, double *gap) {
  const int64_t H = d->H;
  or_route(d, router, x, T, ids, w, logits, gap);
  double *xd = (double *)malloc(sizeof(double) * H);
  double *ye = (double *)malloc(sizeof(double) * H);
  for (int32_t t = 0; t < T; ++t) {
    double *yt = y + (int64_t)t * H;
    for (int64_t j = 0; j < H; ++j) {
      yt[j] = 0.0;
      xd[j] = or_bf16(x[(int64_t)t * H + j]);
    }
    for (int k = 0; k < d->K; ++k) {
      int32_t e = ids[(int64_t)t * d->K + k];
      if (!blobs[e]) {
        fprintf(stderr, "oracle: blob of selected expert %d not provided\n", e);
        abort();
      }
      or_expert(d, blobs[e], xd, ye, NULL);
      const double wk = w[(int64_t)t * d->K + k];
      for (int64_t j = 0; j < H; ++j) yt[j] += wk * ye[j];
    }
    if (d->has_shared) {
      or_expert(d, shared, xd, ye, NULL);
      for (int64_t j = 0; j < H; ++j) yt[j] += ye[j];
    }
  }
  free(xd);
  free(ye);
}

/* Expert forward with routing given (ids/w as doubles per slot). */
void or_expert_forward(const or_dims *d, const uint8_t *const *blobs, const uint8_t *shared,
                       const uint16_t *x, int32_t T, const int32_t *ids, const double *w,
                       double *y) {
  const int64_t H = d->H;
  double *xd = (double *)malloc(sizeof(double) * H);
  double *ye = (double *)malloc(sizeof(double) * H);
  for (int32_t t = 0; t < T; ++t) {
    double *yt = y + (int64_t)t * H;
    for (int64_t j = 0; j < H; ++j) {
      yt[j] = 0.0;
      xd[j] = or_bf16(x[(int64_t)t * H + j]);
    }
    for (int k = 0; k < d->K; ++k) {
      int32_t e = ids[(int64_t)t * d->K + k];
      if (e < 0 || e >= d->E) continue; /* an invalid id contributes 0 */
      if (!blobs[e]) {
        fprintf(stderr, "oracle: blob of selected expert %d not provided\n", e);
        abort();
      }
      or_expert(d, blobs[e], xd, ye, NULL);
      for (int64_t j = 0; j < H; ++j) yt[j] += w[(int64_t)t * d->K + k] * ye[j];
    }
    if (d->has_shared) {
      or_expert(d, shared, xd, ye, NULL);
      for (int64_t j = 0; j < H; ++j) yt[j] += ye[j];
    }
  }
  free(xd);
  free(ye);
}

/* ---- residual stream and pre-MoE norm --------------------------------------
 * "Flash-MoE: Running a 397B Parameter Model on a Laptop" (hysenlabs.com),
 * section "How the SSD expert streaming pipeline works": the layer's last
 * command does the expert forward "plus combine and norm".  Reading taken:
 * the MoE output is added to an fp32 residual stream r, and the next MoE
 * input is its RMS normalisation without a gain,
 *     x_c = r_c / sqrt(mean_c r_c^2 + 1e-6),
 * rounded to bf16 (the MoE input format). */

/* Round a double to the nearest bf16 (ties to even), in one step from the
 * double.  bf16 keeps the sign, the 8 exponent bits of fp32 and 8 significant
 * bits: a value with binary exponent E (2^E <= |v| < 2^(E+1)) is a multiple
 * of 2^(E-7) when normal, and every subnormal is a multiple of 2^-133.  So v
 * is scaled to units of that quantum (exact: a power of two), rounded to the
 * nearest integer with ties to even (rint in the default rounding mode), and
 * scaled back; the result is a bf16 value, so its conversion to float is
 * exact and its upper 16 bits are the pattern.  Magnitudes that round to
 * 2^128 or beyond give infinity. */
uint16_t or_f64_to_bf16(double v) {
  double r = 0.0;
  if (v != 0.0) {
    int e;
    frexp(v, &e); /* |v| = m 2^e, 0.5 <= m < 1, so the exponent E is e - 1 */
    int qexp = (e - 1) - 7;
    if (qexp < -133) qexp = -133;
    r = ldexp(rint(ldexp(v, -qexp)), qexp);
  }
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (fabs(r) >= 0x1p128) return (uint16_t)(sign | 0x7F80u);
  float f = (float)r;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u >> 16) | sign);
}

/* x = bf16(r / sqrt(mean(r^2) + eps)) for one token of n values. */
void or_rmsnorm_bf16(int64_t n, const float *r, double eps, uint16_t *x) {
  double ss = 0.0;
  for (int64_t c = 0; c < n; ++c) ss += (double)r[c] * (double)r[c];
  const double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t c = 0; c < n; ++c) x[c] = or_f64_to_bf16((double)r[c] * inv);
}

/* One layer on the residual stream for T tokens: x = rmsnorm(r) (bf16),
 * y = layer(x), r_out = r + y.  Outputs as or_layer, plus x [T][H] and
 * r_out [T][H] (double). */
void or_residual_layer(const or_dims *d, const uint16_t *router, const uint8_t *const *blobs,
                       const uint8_t *shared, const float *r, int32_t T, double *r_out,
                       uint16_t *x, double *y, int32_t *ids, double *w, double *logits,
                       double *gap) {
  const int64_t H = d->H;
  for (int32_t t = 0; t < T; ++t) or_rmsnorm_bf16(H, r + (int64_t)t * H, 1e-6, x + (int64_t)t * H);
  or_layer(d, router, blobs, shared, x, T, y, ids, w, logits, gap);
  for (int64_t i = 0; i < (int64_t)T * H; ++i) r_out[i] = (double)r[i] + y[i];
}

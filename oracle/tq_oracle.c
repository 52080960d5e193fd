/*
 * tq_oracle.c -- CPU oracle for the TurboQuant KV-cache path.
 *
 * TEST INFRASTRUCTURE ONLY (see tq_oracle.h).  Plain single-threaded C99,
 * compiled with -O2 -ffp-contract=off and no fast-math, so every expression
 * is evaluated exactly as written.
 *
 * Parity status per function (the pins live in tests/test_oracle_*.py):
 *   fp16 conversion ......... pinned (numpy float16, exhaustive over a grid)
 *   SplitMix64 .............. pinned (published reference outputs)
 *   signs / Gaussian sketch . pinned statistically (balance, moments, KS)
 *   codebook ................ pinned (Lloyd conditions by scipy quadrature,
 *                             Max (1960) Gaussian limit, 1-bit closed form)
 *   FWHT .................... pinned (dense Sylvester matrix, H.H = d.I)
 *   quantisers .............. pinned (brute-force nearest centroid, MSE vs
 *                             Lloyd MSE, q8 exact multiples)
 *   QJL estimator ........... pinned (unbiasedness over 10^4 seeds,
 *                             variance closed form)
 *   pack / unpack ........... pinned (round trip, byte counts = closed form)
 *   decode .................. pinned (bypass codec = textbook softmax
 *                             attention, one-token and equal-logit cases)
 */
#include "tq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ===================================================================== */
/* fp16                                                                  */
/* ===================================================================== */

uint16_t or_f32_to_f16(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) {                 /* inf or NaN */
    return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
  }
  if (ax >= 0x477ff000u) {                 /* >= 65520 rounds to infinity */
    return (uint16_t)(sign | 0x7c00u);
  }
  if (ax < 0x38800000u) {                  /* below 2^-14: fp16 subnormal or zero */
    float v;
    memcpy(&v, &ax, 4);
    float scaled = v * 16777216.0f;        /* v / 2^-24, exact (power of two) */
    float r = rintf(scaled);               /* round half to even */
    return (uint16_t)(sign | (uint32_t)r); /* r == 1024 is the smallest normal */
  }
  uint32_t e = (ax >> 23) - 127u + 15u;
  uint32_t mant = ax & 0x7fffffu;
  uint32_t h = (e << 10) | (mant >> 13);
  uint32_t rem = mant & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;  /* carry may bump the exponent */
  return (uint16_t)(sign | h);
}

float or_f16_to_f32(uint16_t h) {
  uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1fu;
  uint32_t mant = h & 0x3ffu;
  float v;
  if (e == 0) {
    v = (float)mant * (1.0f / 16777216.0f);  /* subnormal: mant * 2^-24, exact */
    uint32_t bits;
    memcpy(&bits, &v, 4);
    bits |= sign;
    memcpy(&v, &bits, 4);
    return v;
  }
  uint32_t bits;
  if (e == 31) {
    bits = sign | 0x7f800000u | (mant << 13);
  } else {
    bits = sign | ((e - 15u + 127u) << 23) | (mant << 13);
  }
  memcpy(&v, &bits, 4);
  return v;
}

void or_f32_to_f16_array(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = or_f32_to_f16(x[i]);
}
void or_f16_to_f32_array(const uint16_t* x, float* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = or_f16_to_f32(x[i]);
}

/* Norm fields are non-negative; values beyond the fp16 range saturate. */
uint16_t or_norm_to_f16(float n) {
  return or_f32_to_f16(n < 65504.0f ? n : 65504.0f);
}

/* ===================================================================== */
/* SplitMix64, counter form                                              */
/* ===================================================================== */

#define OR_GOLDEN 0x9E3779B97F4A7C15ULL

uint64_t or_splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* The generator adds the golden gamma to its state before mixing, so the
 * k-th output (0-based) of a generator started at s0 mixes s0 + (k+1)*gamma. */
uint64_t or_splitmix64_at(uint64_t s0, uint64_t k) {
  return or_splitmix64_mix(s0 + (k + 1u) * OR_GOLDEN);
}

uint64_t or_stream_u64(uint64_t seed, int32_t layer, uint32_t stream, uint64_t k) {
  uint64_t key = or_splitmix64_at(seed, ((uint64_t)(uint32_t)layer << 8) + (uint64_t)stream);
  return or_splitmix64_at(key, k);
}

/* Reading: D_i = -1 when the top bit of value i is set, else +1. */
void or_make_signs(uint64_t seed, int32_t layer, uint32_t stream, int d, float* D) {
  for (int i = 0; i < d; i++) {
    D[i] = (or_stream_u64(seed, layer, stream, (uint64_t)i) >> 63) ? -1.0f : 1.0f;
  }
}

/* Reading: S[j][i] (row j of m, column i of d) uses values 2e and 2e+1 of
 * stream 2, e = j*d + i: u1 in (0,1], u2 in [0,1), g = sqrt(-2 ln u1) cos(2 pi u2),
 * computed in fp64 and rounded once to fp32. */
void or_make_sketch(uint64_t seed, int32_t layer, int m, int d, float* S) {
  const double two_pi = 6.283185307179586;   /* 2*pi rounded to double */
  const double inv53 = 1.0 / 9007199254740992.0;
  for (int j = 0; j < m; j++) {
    for (int i = 0; i < d; i++) {
      uint64_t e = (uint64_t)j * (uint64_t)d + (uint64_t)i;
      uint64_t a = or_stream_u64(seed, layer, 2u, 2u * e);
      uint64_t c = or_stream_u64(seed, layer, 2u, 2u * e + 1u);
      double u1 = (double)((a >> 11) + 1u) * inv53;
      double u2 = (double)(c >> 11) * inv53;
      double g = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
      S[(size_t)j * d + i] = (float)g;
    }
  }
}

/* ===================================================================== */
/* Codebook                                                              */
/* ===================================================================== */

/* Reading: a uniformly random unit vector u in R^d has coordinates with
 * density prop. to (1 - u^2)^((d-3)/2); the rotated coordinate divided by the
 * vector norm is t = sqrt(d) u, with density prop. to (1 - t^2/d)^((d-3)/2)
 * on |t| < sqrt(d).  Beyond |t| = 16 the weight is below e^-120 of its
 * peak (for every d >= 128) and is taken as zero. */
static double or_weight(int d, double t) {
  double v = 1.0 - t * t / (double)d;
  if (v <= 0.0) return 0.0;
  return pow(v, 0.5 * (double)(d - 3));
}

static double or_tmax(int d) {
  double r = sqrt((double)d);
  return r < 16.0 ? r : 16.0;
}

#define OR_SIMPSON_N 4096   /* even number of sub-intervals per integral */

static double or_simpson(int d, double a, double c, int moment) {
  if (c <= a) return 0.0;
  double h = (c - a) / OR_SIMPSON_N;
  double acc = 0.0;
  for (int k = 0; k <= OR_SIMPSON_N; k++) {
    double t = a + h * k;
    double f = or_weight(d, t);
    if (moment == 1) f *= t;
    if (moment == 2) f *= t * t;
    double wk = (k == 0 || k == OR_SIMPSON_N) ? 1.0 : ((k & 1) ? 4.0 : 2.0);
    acc += wk * f;
  }
  return acc * h / 3.0;
}

double or_marginal_mass(int d, double a, double c) { return or_simpson(d, a, c, 0); }
double or_marginal_moment1(int d, double a, double c) { return or_simpson(d, a, c, 1); }

/* Lloyd-Max (alternate: boundaries at midpoints of centroids, centroids at
 * the conditional mean of their cell) in fp64.  The density is symmetric,
 * so the optimum for 2^b levels is symmetric with a boundary at 0; only the
 * positive half (K = 2^(b-1) levels) is iterated and then mirrored.  Stop
 * when no centroid moves by more than 1e-13 (the quadrature's noise floor
 * is near 1e-15), or after 100000 rounds. */
int or_codebook(int d, int b, double* cent64, uint16_t* c16, float* bounds, double* mse) {
  if (d < 4 || b < 1 || b > 8) return -1;
  int L = 1 << b;
  int K = L / 2;
  double tmax = or_tmax(d);
  double* c = (double*)malloc(sizeof(double) * K);
  double* e = (double*)malloc(sizeof(double) * (K + 1));   /* cell edges, e[0] = 0 */
  for (int k = 0; k < K; k++) c[k] = 3.0 * (k + 0.5) / K;
  int it;
  for (it = 1; it <= 100000; it++) {
    e[0] = 0.0;
    for (int k = 1; k < K; k++) e[k] = 0.5 * (c[k - 1] + c[k]);
    e[K] = tmax;
    double moved = 0.0;
    for (int k = 0; k < K; k++) {
      double m0 = or_simpson(d, e[k], e[k + 1], 0);
      double m1 = or_simpson(d, e[k], e[k + 1], 1);
      double nc = m1 / m0;
      double dd = fabs(nc - c[k]);
      if (dd > moved) moved = dd;
      c[k] = nc;
    }
    if (moved <= 1e-13) break;
  }
  /* mirror: index 0 is the most negative level */
  for (int k = 0; k < K; k++) {
    cent64[K + k] = c[k];
    cent64[K - 1 - k] = -c[k];
  }
  for (int j = 0; j < L; j++) c16[j] = or_f32_to_f16((float)cent64[j]);
  /* note: (float)cent64 then RNE to fp16 is a double rounding; the tests
   * check that every centroid lies far from an fp16 rounding tie, where the
   * double rounding equals a single rounding. */
  for (int j = 0; j + 1 < L; j++) {
    float lo = or_f16_to_f32(c16[j]);
    float hi = or_f16_to_f32(c16[j + 1]);
    bounds[j] = (lo + hi) * 0.5f;   /* exact: fp16 values summed in fp32 */
  }
  if (mse) {
    e[0] = 0.0;
    for (int k = 1; k < K; k++) e[k] = 0.5 * (c[k - 1] + c[k]);
    e[K] = tmax;
    double num = 0.0, den = or_simpson(d, 0.0, tmax, 0);
    for (int k = 0; k < K; k++) {
      double m0 = or_simpson(d, e[k], e[k + 1], 0);
      double m1 = or_simpson(d, e[k], e[k + 1], 1);
      double m2 = or_simpson(d, e[k], e[k + 1], 2);
      num += m2 - 2.0 * c[k] * m1 + c[k] * c[k] * m0;
    }
    *mse = num / den;
  }
  free(c);
  free(e);
  return it;
}

/* ===================================================================== */
/* Rotation and norms                                                    */
/* ===================================================================== */

/* Reading: unnormalised Sylvester-ordered Walsh-Hadamard transform,
 * stages h = 1, 2, 4, ..., d/2; butterfly (a, b) -> (a + b, a - b) on the pair
 * (j, j + h) with bit h of j clear. */
void or_fwht_f32(float* x, int d) {
  for (int h = 1; h < d; h *= 2) {
    for (int i = 0; i < d; i += 2 * h) {
      for (int j = i; j < i + h; j++) {
        float a = x[j];
        float b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
    }
  }
}

void or_fwht_f64(double* x, int d) {
  for (int h = 1; h < d; h *= 2) {
    for (int i = 0; i < d; i += 2 * h) {
      for (int j = i; j < i + h; j++) {
        double a = x[j];
        double b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
    }
  }
}

/* Reading: the sum of squares is taken in fp64 (each square of an fp32
 * value is exact in fp64) as a pairwise tree: s_i = x_i^2, then for
 * w = d/2, d/4, ..., 1: s_i += s_{i+w} for i < w; the total is s_0. */
double or_tree_sumsq_f32(const float* x, int d) {
  double* s = (double*)malloc(sizeof(double) * d);
  for (int i = 0; i < d; i++) s[i] = (double)x[i] * (double)x[i];
  for (int w = d / 2; w >= 1; w /= 2) {
    for (int i = 0; i < w; i++) s[i] = s[i] + s[i + w];
  }
  double r = s[0];
  free(s);
  return r;
}

/* ===================================================================== */
/* Quantisers                                                            */
/* ===================================================================== */

/* One vector, POLAR or POLAR_QJL ([P1] PolarQuant and QJL paragraphs).
 *  y      = H (D . x)                       fp32, exact butterfly order
 *  n      = fp32(sqrt(tree sum x^2))        radius 
 *  n16    = fp16(min(n, 65504))             stored radius
 *  code_i = #{ j : y_i > fp32(B_j * n) }    angle code (nearest fp16 centroid
 *                                           of t_i = y_i / n, ties go low)
 * QJL :
 *  r_i    = fmaf(-n16, C[code_i], y_i)      rotated-frame residual
 *  rho    = fp32(sqrt(tree sum r^2 / d))    = |x - x_hat| in the input frame
 *  z_j    = sum_i S[j][i] r_i               fp64, sequential
 *  sign_j = (z_j >= 0)                      1 bit per sketch row
 */
void or_quantize_polar(const float* x, int d, int b, const float* D,
                       const uint16_t* c16, const float* bounds,
                       int m, const float* S,
                       uint8_t* codes, uint16_t* n16, uint8_t* signs, uint16_t* rho16,
                       double* tmargin, double* z, double* rrot) {
  int L = 1 << b;
  float* y = (float*)malloc(sizeof(float) * d);
  for (int i = 0; i < d; i++) y[i] = D[i] * x[i];
  or_fwht_f32(y, d);
  double s = or_tree_sumsq_f32(x, d);
  float n = (float)sqrt(s);
  uint16_t nh = or_norm_to_f16(n);
  *n16 = nh;
  for (int i = 0; i < d; i++) {
    int c = 0;
    for (int j = 0; j + 1 < L; j++) {
      float thr = bounds[j] * n;
      if (y[i] > thr) c++;
    }
    codes[i] = (uint8_t)c;
    if (tmargin) {
      double best = 1e300;
      if (n > 0.0f) {
        double t = (double)y[i] / (double)n;
        for (int j = 0; j + 1 < L; j++) {
          double dd = fabs(t - (double)bounds[j]);
          if (dd < best) best = dd;
        }
      }
      tmargin[i] = best;
    }
  }
  if (m > 0 && S != NULL) {
    float nf = or_f16_to_f32(nh);
    float* r = (float*)malloc(sizeof(float) * d);
    for (int i = 0; i < d; i++) r[i] = fmaf(-nf, or_f16_to_f32(c16[codes[i]]), y[i]);
    double sr = or_tree_sumsq_f32(r, d);
    float rho = (float)sqrt(sr / (double)d);
    *rho16 = or_norm_to_f16(rho);
    if (rrot) *rrot = sqrt(sr);
    for (int j = 0; j < m; j++) {
      double acc = 0.0;
      for (int i = 0; i < d; i++) acc += (double)S[(size_t)j * d + i] * (double)r[i];
      signs[j] = (uint8_t)(acc >= 0.0 ? 1 : 0);
      if (z) z[j] = acc;
    }
    free(r);
  }
  free(y);
}

/* Reading: blocks of 32 consecutive unrotated coordinates;
 * s = amax/127 (fp32), s16 = fp16(s), k = clamp(rint(x / s16), -127, 127)
 * with a correctly rounded fp32 division; s16 == 0 gives all-zero codes. */
void or_quantize_q8(const float* x, int d, int8_t* k8, uint16_t* s16, double* qmargin) {
  for (int blk = 0; blk < d / 32; blk++) {
    float amax = 0.0f;
    for (int i = blk * 32; i < blk * 32 + 32; i++) {
      float a = fabsf(x[i]);
      if (a > amax) amax = a;
    }
    float sc = amax / 127.0f;
    uint16_t sh = or_norm_to_f16(sc);
    s16[blk] = sh;
    float sf = or_f16_to_f32(sh);
    for (int i = blk * 32; i < blk * 32 + 32; i++) {
      int k = 0;
      double mg = 1e300;
      if (sf > 0.0f) {
        float q = x[i] / sf;
        float r = rintf(q);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        k = (int)r;
        double fl = floor((double)q);
        mg = fabs((double)q - (fl + 0.5));
      }
      k8[i] = (int8_t)k;
      if (qmargin) qmargin[i] = mg;
    }
  }
}

/* ===================================================================== */
/* Dequantisers (fp64)                                                   */
/* ===================================================================== */

/* x_hat = D . H (n16 C[code]) / d  (H H = d I, so H/d inverts the raw H). */
void or_dequant_polar(int d, const float* D, const uint16_t* c16,
                      const uint8_t* codes, uint16_t n16, double* out) {
  double n = (double)or_f16_to_f32(n16);
  for (int i = 0; i < d; i++) out[i] = n * (double)or_f16_to_f32(c16[codes[i]]);
  or_fwht_f64(out, d);
  for (int i = 0; i < d; i++) out[i] = (double)D[i] * out[i] / (double)d;
}

/* x_tilde = x_hat + rho sqrt(pi/2)/m R^T S^T sigma, R^T = D H / sqrt(d),
 * sigma_j = +1 for a set bit and -1 otherwise.  <q, x_tilde> equals the
 * QJL-corrected estimator of <q, x>. */
void or_dequant_polar_qjl(int d, int m, const float* D, const uint16_t* c16, const float* S,
                          const uint8_t* codes, uint16_t n16, const uint8_t* signs,
                          uint16_t rho16, double* out) {
  or_dequant_polar(d, D, c16, codes, n16, out);
  double* u = (double*)malloc(sizeof(double) * d);
  for (int i = 0; i < d; i++) {
    double acc = 0.0;
    for (int j = 0; j < m; j++) {
      double sg = signs[j] ? 1.0 : -1.0;
      acc += (double)S[(size_t)j * d + i] * sg;
    }
    u[i] = acc;
  }
  or_fwht_f64(u, d);
  double rho = (double)or_f16_to_f32(rho16);
  double k = rho * sqrt(M_PI / 2.0) / (double)m / sqrt((double)d);
  for (int i = 0; i < d; i++) out[i] += k * (double)D[i] * u[i];
  free(u);
}

void or_dequant_q8(int d, const int8_t* k8, const uint16_t* s16, double* out) {
  for (int i = 0; i < d; i++) out[i] = (double)or_f16_to_f32(s16[i / 32]) * (double)k8[i];
}

/* ===================================================================== */
/* Recursive polar codec (POLAR_TREE)                                    */
/* ===================================================================== */
/*
 * [P1]'s Cartesian-to-polar paragraph read literally: the rotated vector y
 * (d = 2^L coordinates) is rewritten as one radius and d - 1 angles by
 * pairing recursively.  Level 1 pairs the coordinates (y_2i, y_2i+1): angle
 * atan2(y_2i+1, y_2i) in [0, 2 pi).  Level l >= 2 pairs the radii of two
 * sibling nodes of level l - 1: angle atan2(r_right, r_left) in [0, pi/2].
 * The last radius is |y|.  For a spherically symmetric y the angles are
 * independent, level 1 uniform on the circle and level l distributed with
 * density prop. to sin(2 theta)^(2^(l-1) - 1) on [0, pi/2] (the squared
 * radii of the two halves are chi-square with 2^(l-1) degrees each) -- the
 * "distribution known in advance" of the paragraph.
 *
 * Angles live in heap slots: the node at slot s (1 <= s < d) has children
 * 2s and 2s + 1, slots d .. 2d - 1 being the coordinates y_0 .. y_d-1.  So
 * slot d/2 + i is level-1 pair i, slot 2^(L-l) + k is node k of level l, slot
 * 1 is the root, slot 0 is unused.
 *
 * Reading of the bit budget (the pages give none): with b bits per
 * coordinate, level 1 angles take b + 1 bits and every other angle b - 1
 * bits, (d/2)(b + 1) + (d/2 - 1)(b - 1) = d b - 1 bits, plus the fp16 radius:
 * the same record size as the per-coordinate codec with b bits.  Level 1 uses
 * the uniform quantiser of the circle (cells [2 pi j / 2^(b+1), 2 pi (j+1) /
 * 2^(b+1)], centroid at the middle); higher levels a Lloyd-Max codebook for
 * their density.  Decisions: code = #{ boundaries below the angle } (ties go
 * to the lower cell), angles from fp64 atan2 of fp64 coordinates and radii.
 */

static int or_tree_levels(int d) {
  int L = 0;
  while ((1 << L) < d) L++;
  return L;
}

/* level of heap slot s (1 <= s < d) */
static int or_slot_level(int d, int s) {
  int L = or_tree_levels(d), k = 0;
  while ((2 << k) <= s) k++;   /* k = floor(log2 s) */
  return L - k;
}

static double or_angle_weight(int level, double th) {
  double v = sin(2.0 * th);
  if (v <= 0.0) return 0.0;
  return pow(v, (double)((1 << (level - 1)) - 1));
}

static double or_angle_simpson(int level, double a, double c, int moment) {
  if (c <= a) return 0.0;
  double h = (c - a) / OR_SIMPSON_N;
  double acc = 0.0;
  for (int k = 0; k <= OR_SIMPSON_N; k++) {
    double t = a + h * k;
    double f = or_angle_weight(level, t);
    if (moment == 1) f *= t;
    if (moment == 2) f *= t * t;
    double wk = (k == 0 || k == OR_SIMPSON_N) ? 1.0 : ((k & 1) ? 4.0 : 2.0);
    acc += wk * f;
  }
  return acc * h / 3.0;
}

double or_angle_mass(int level, double a, double c) { return or_angle_simpson(level, a, c, 0); }
double or_angle_moment1(int level, double a, double c) { return or_angle_simpson(level, a, c, 1); }

/* Codebook of the level-`level` angle with `bits` bits: cent[2^bits] in
 * increasing order, bounds[2^bits - 1] (midpoints), *mse = E[(theta -
 * Q(theta))^2] under the level's law.  Level 1: uniform quantiser of [0, 2 pi).
 * Level >= 2: Lloyd-Max, symmetric about pi/4 (the density is), iterated on
 * [0, pi/4] until no centroid moves by more than 1e-13.  Returns the number
 * of Lloyd rounds (0 for level 1), or -1 on bad arguments. */
int or_angle_codebook(int level, int bits, double* cent, double* bounds, double* mse) {
  if (level < 1 || level > 12 || bits < 1 || bits > 8) return -1;
  int n = 1 << bits;
  if (level == 1) {
    double w = 2.0 * M_PI / n;
    for (int j = 0; j < n; j++) cent[j] = (j + 0.5) * w;
    for (int j = 0; j + 1 < n; j++) bounds[j] = (j + 1) * w;
    if (mse) *mse = w * w / 12.0;
    return 0;
  }
  int K = n / 2;
  double q = M_PI / 4.0;
  double* c = (double*)malloc(sizeof(double) * K);
  double* e = (double*)malloc(sizeof(double) * (K + 1));
  for (int k = 0; k < K; k++) c[k] = q * (k + 0.5) / K;
  int it;
  for (it = 1; it <= 100000; it++) {
    e[0] = 0.0;
    for (int k = 1; k < K; k++) e[k] = 0.5 * (c[k - 1] + c[k]);
    e[K] = q;
    double moved = 0.0;
    for (int k = 0; k < K; k++) {
      double nc = or_angle_simpson(level, e[k], e[k + 1], 1) / or_angle_simpson(level, e[k], e[k + 1], 0);
      if (fabs(nc - c[k]) > moved) moved = fabs(nc - c[k]);
      c[k] = nc;
    }
    if (moved <= 1e-13) break;
  }
  for (int k = 0; k < K; k++) {
    cent[k] = c[k];
    cent[n - 1 - k] = 2.0 * q - c[k];
  }
  for (int j = 0; j + 1 < n; j++) bounds[j] = 0.5 * (cent[j] + cent[j + 1]);
  bounds[K - 1] = q;
  if (mse) {
    double num = 0.0, den = or_angle_simpson(level, 0.0, q, 0);
    e[0] = 0.0;
    for (int k = 1; k < K; k++) e[k] = 0.5 * (c[k - 1] + c[k]);
    e[K] = q;
    for (int k = 0; k < K; k++) {
      double m0 = or_angle_simpson(level, e[k], e[k + 1], 0);
      double m1 = or_angle_simpson(level, e[k], e[k + 1], 1);
      double m2 = or_angle_simpson(level, e[k], e[k + 1], 2);
      num += m2 - 2.0 * c[k] * m1 + c[k] * c[k] * m0;
    }
    *mse = num / den;
  }
  free(c);
  free(e);
  return it;
}

/* Angles of y (fp64) in heap slots ang[1..d-1]; returns |y|.  Signed zeros
 * are read as +0. */
double or_tree_angles(const double* y, int d, double* ang) {
  double* r2 = (double*)malloc(sizeof(double) * 2 * d);
  for (int i = 0; i < d; i++) r2[d + i] = y[i] * y[i];
  for (int s = d - 1; s >= 1; s--) r2[s] = r2[2 * s] + r2[2 * s + 1];
  ang[0] = 0.0;
  for (int s = 1; s < d; s++) {
    if (s >= d / 2) {
      double a = y[2 * s - d] + 0.0, b = y[2 * s + 1 - d] + 0.0;
      double th = atan2(b, a);
      if (th < 0.0) th += 2.0 * M_PI;
      ang[s] = th;
    } else {
      ang[s] = atan2(sqrt(r2[2 * s + 1]), sqrt(r2[2 * s]));
    }
  }
  double r = sqrt(r2[1]);
  free(r2);
  return r;
}

/* Inverse of or_tree_angles: y from the radius r and the angles. */
void or_tree_from_angles(const double* ang, double r, int d, double* y) {
  double* rad = (double*)malloc(sizeof(double) * 2 * d);
  rad[1] = r;
  for (int s = 1; s < d; s++) {
    rad[2 * s] = rad[s] * cos(ang[s]);
    rad[2 * s + 1] = rad[s] * sin(ang[s]);
  }
  for (int i = 0; i < d; i++) y[i] = rad[d + i];
  free(rad);
}

void or_tree_tables(int d, int b, or_tree_tab* T) {
  int L = or_tree_levels(d);
  T->d = d;
  T->b = b;
  T->levels = L;
  for (int l = 1; l <= L; l++) {
    T->bits[l] = (l == 1) ? b + 1 : b - 1;
    or_angle_codebook(l, T->bits[l], T->cent[l], T->bnd[l], NULL);
  }
}

/* One vector: y = H (D . x) in fp32 as for POLAR, n16 as for POLAR, then the
 * angles of y (fp64) and per slot the code #{ j : B_j < angle }.  amargin
 * (optional, [d]) gets the distance of each angle to the nearest decision
 * boundary, the wrap-around at 0 = 2 pi included for level 1. */
void or_quantize_tree(const float* x, int d, const float* D, const or_tree_tab* T,
                      uint8_t* codes, uint16_t* n16, double* amargin) {
  float* y = (float*)malloc(sizeof(float) * d);
  double* yd = (double*)malloc(sizeof(double) * d);
  double* ang = (double*)malloc(sizeof(double) * d);
  for (int i = 0; i < d; i++) y[i] = D[i] * x[i];
  or_fwht_f32(y, d);
  double s = or_tree_sumsq_f32(x, d);
  *n16 = or_norm_to_f16((float)sqrt(s));
  for (int i = 0; i < d; i++) yd[i] = (double)y[i];
  or_tree_angles(yd, d, ang);
  codes[0] = 0;
  if (amargin) amargin[0] = 1e300;
  for (int sl = 1; sl < d; sl++) {
    int l = or_slot_level(d, sl);
    int nb = 1 << T->bits[l];
    int c = 0;
    double mg = 1e300;
    for (int j = 0; j + 1 < nb; j++) {
      if (ang[sl] > T->bnd[l][j]) c++;
      double dd = fabs(ang[sl] - T->bnd[l][j]);
      if (dd < mg) mg = dd;
    }
    if (l == 1) {
      if (ang[sl] < mg) mg = ang[sl];
      if (2.0 * M_PI - ang[sl] < mg) mg = 2.0 * M_PI - ang[sl];
    }
    codes[sl] = (uint8_t)c;
    if (amargin) amargin[sl] = mg;
  }
  free(ang);
  free(yd);
  free(y);
}

/* x_hat = D . H (sqrt(d) n16 u) / d, u the unit vector whose angles are the
 * code centroids (H H = d I). */
void or_dequant_tree(int d, const float* D, const or_tree_tab* T, const uint8_t* codes,
                     uint16_t n16, double* out) {
  double* ang = (double*)malloc(sizeof(double) * d);
  ang[0] = 0.0;
  for (int sl = 1; sl < d; sl++) ang[sl] = T->cent[or_slot_level(d, sl)][codes[sl]];
  or_tree_from_angles(ang, sqrt((double)d) * (double)or_f16_to_f32(n16), d, out);
  or_fwht_f64(out, d);
  for (int i = 0; i < d; i++) out[i] = (double)D[i] * out[i] / (double)d;
  free(ang);
}

/* Tables for the whole-cache helpers, one per b = 2..4 at d = 128, built by
 * or_tree_prepare before any other call uses them. */
static or_tree_tab or_tree_cache[5];
static int or_tree_ready = 0;

void or_tree_prepare(void) {
  if (or_tree_ready) return;
  for (int b = 2; b <= 4; b++) or_tree_tables(128, b, &or_tree_cache[b]);
  or_tree_ready = 1;
}

const or_tree_tab* or_tree_table(int b) {
  if (!or_tree_ready || b < 2 || b > 4) return NULL;
  return &or_tree_cache[b];
}

/* ===================================================================== */
/* Layout                                                                */
/* ===================================================================== */
/*
 * Cache image: [batch][n_kv][n_blocks][block], n_blocks = ceil(max_ctx/128),
 * block = 128 consecutive positions of one (sequence, kv head).
 *
 * Inside a block, the per-position fields of POLAR / POLAR_QJL keys (code
 * words, sign words, radius, residual norm) and the radius of POLAR values
 * sit at slot pi(t) = 32 (t/32) + 8 (t%4) + (t%32)/4 for position t (a
 * fixed permutation inside each group of 32 positions).
 *
 * K block, POLAR / POLAR_QJL with b bits, m sketch rows:
 *   plane p (p < b):  u32 word[d/32][128]; word[j][pi(t)] bit e = bit p of
 *                     the code of coordinate 32 j + e of token t
 *   sign plane (QJL): u32 word[m/32][128]; bit e of word[j][pi(t)] = sign bit
 *                     of sketch row 32 j + e of token t
 *   n16[128]  fp16;   rho16[128] fp16 (QJL), both at slot pi(t)
 * K block, Q8:   int8 k8[128][d], then fp16 s16[128][d/32]
 * K/V block RAW: fp32 [128][d]
 * V block, POLAR with b bits:
 *   plane p:          u32 word[4][d]; bit e of word[j][i] = bit p of the code
 *                     of coordinate i of token 32 j + e (natural order)
 *   n16[128] fp16 at slot pi(t)
 * K block, POLAR_TREE with b bits (angle slots a = 0..d-1, slot 0 unused):
 *   plane p < b - 1:  u32 word[d/32][128]; bit e of word[j][pi(t)] = bit p of
 *                     the code of angle slot 32 j + e of token t
 *   2 level-1 planes: u32 word[d/64][128]; bit e of word[j][pi(t)] = bit
 *                     b - 1 + x (plane x) of the code of slot d/2 + 32 j + e
 *   n16[128] fp16 at slot pi(t)
 * V block, POLAR_TREE with b bits:
 *   plane p < b - 1:  u32 word[4][d]; bit e of word[j][a] = bit p of the code
 *                     of angle slot a of token 32 j + e
 *   2 level-1 planes: u32 word[4][d/2]; bit e of word[j][a - d/2] = bit
 *                     b - 1 + x of the code of slot a of token 32 j + e
 *   n16[128] fp16 at slot pi(t)
 */

static int or_nblocks(const or_spec* s) { return (s->max_ctx + OR_BLOCK - 1) / OR_BLOCK; }

int64_t or_k_record_bytes(const or_spec* s) {
  switch (s->k_codec) {
    case OR_RAW_F32: return 4 * (int64_t)s->d;
    case OR_POLAR:
    case OR_POLAR_TREE: return (int64_t)s->k_bits * s->d / 8 + 2;
    case OR_POLAR_QJL: return (int64_t)s->k_bits * s->d / 8 + s->m / 8 + 4;
    case OR_Q8_BLOCK32: return (int64_t)s->d + 2 * (s->d / 32);
  }
  return -1;
}
int64_t or_v_record_bytes(const or_spec* s) {
  switch (s->v_codec) {
    case OR_RAW_F32: return 4 * (int64_t)s->d;
    case OR_POLAR:
    case OR_POLAR_TREE: return (int64_t)s->v_bits * s->d / 8 + 2;
  }
  return -1;
}
int64_t or_k_block_bytes(const or_spec* s) { return OR_BLOCK * or_k_record_bytes(s); }
int64_t or_v_block_bytes(const or_spec* s) { return OR_BLOCK * or_v_record_bytes(s); }
int64_t or_k_cache_bytes(const or_spec* s) {
  return (int64_t)s->batch * s->n_kv * or_nblocks(s) * or_k_block_bytes(s);
}
int64_t or_v_cache_bytes(const or_spec* s) {
  return (int64_t)s->batch * s->n_kv * or_nblocks(s) * or_v_block_bytes(s);
}

static uint8_t* or_kblock(const or_spec* s, int b, int pos, int h, uint8_t* kc) {
  int64_t blk = ((int64_t)b * s->n_kv + h) * or_nblocks(s) + pos / OR_BLOCK;
  return kc + blk * or_k_block_bytes(s);
}
static uint8_t* or_vblock(const or_spec* s, int b, int pos, int h, uint8_t* vc) {
  int64_t blk = ((int64_t)b * s->n_kv + h) * or_nblocks(s) + pos / OR_BLOCK;
  return vc + blk * or_v_block_bytes(s);
}

static int or_slot(int t) { return 32 * (t / 32) + 8 * (t % 4) + (t % 32) / 4; }

static void or_setbit(uint8_t* base, int64_t word, int bit, int v) {
  uint32_t w;
  memcpy(&w, base + 4 * word, 4);
  if (v) w |= (1u << bit); else w &= ~(1u << bit);
  memcpy(base + 4 * word, &w, 4);
}
static int or_getbit(const uint8_t* base, int64_t word, int bit) {
  uint32_t w;
  memcpy(&w, base + 4 * word, 4);
  return (int)((w >> bit) & 1u);
}

void or_pack_k(const or_spec* s, int b, int pos, int h, const or_krec* r, int64_t rec, uint8_t* kc) {
  uint8_t* blk = or_kblock(s, b, pos, h, kc);
  int t = pos % OR_BLOCK;
  int d = s->d;
  if (s->k_codec == OR_RAW_F32) {
    memcpy(blk + (int64_t)t * d * 4, r->raw + rec * d, 4 * (size_t)d);
    return;
  }
  if (s->k_codec == OR_Q8_BLOCK32) {
    memcpy(blk + (int64_t)t * d, r->k8 + rec * d, (size_t)d);
    uint8_t* sc = blk + (int64_t)OR_BLOCK * d;
    memcpy(sc + (int64_t)t * (d / 32) * 2, r->s16 + rec * (d / 32), 2 * (size_t)(d / 32));
    return;
  }
  int nb = s->k_bits;
  int sl = or_slot(t);
  int64_t plane_words = (int64_t)(d / 32) * OR_BLOCK;
  if (s->k_codec == OR_POLAR_TREE) {
    for (int p = 0; p < nb - 1; p++) {
      for (int a = 0; a < d; a++) {
        int bit = (r->codes[rec * d + a] >> p) & 1;
        or_setbit(blk, p * plane_words + (int64_t)(a / 32) * OR_BLOCK + sl, a % 32, bit);
      }
    }
    uint8_t* l1 = blk + 4 * (nb - 1) * plane_words;
    for (int x = 0; x < 2; x++) {
      for (int a = d / 2; a < d; a++) {
        int bit = (r->codes[rec * d + a] >> (nb - 1 + x)) & 1;
        or_setbit(l1, x * (plane_words / 2) + (int64_t)((a - d / 2) / 32) * OR_BLOCK + sl, a % 32, bit);
      }
    }
    memcpy(l1 + 4 * plane_words + 2 * sl, &r->n16[rec], 2);
    return;
  }
  for (int p = 0; p < nb; p++) {
    for (int i = 0; i < d; i++) {
      int bit = (r->codes[rec * d + i] >> p) & 1;
      or_setbit(blk, p * plane_words + (int64_t)(i / 32) * OR_BLOCK + sl, i % 32, bit);
    }
  }
  uint8_t* after = blk + 4 * nb * plane_words;
  if (s->k_codec == OR_POLAR_QJL) {
    for (int j = 0; j < s->m; j++) {
      or_setbit(after, (int64_t)(j / 32) * OR_BLOCK + sl, j % 32, r->signs[rec * s->m + j]);
    }
    after += 4 * (int64_t)(s->m / 32) * OR_BLOCK;
  }
  memcpy(after + 2 * sl, &r->n16[rec], 2);
  if (s->k_codec == OR_POLAR_QJL) memcpy(after + 2 * OR_BLOCK + 2 * sl, &r->rho16[rec], 2);
}

void or_unpack_k(const or_spec* s, int b, int pos, int h, const uint8_t* kc, or_krec* r, int64_t rec) {
  const uint8_t* blk = or_kblock(s, b, pos, h, (uint8_t*)kc);
  int t = pos % OR_BLOCK;
  int d = s->d;
  if (s->k_codec == OR_RAW_F32) {
    memcpy(r->raw + rec * d, blk + (int64_t)t * d * 4, 4 * (size_t)d);
    return;
  }
  if (s->k_codec == OR_Q8_BLOCK32) {
    memcpy(r->k8 + rec * d, blk + (int64_t)t * d, (size_t)d);
    const uint8_t* sc = blk + (int64_t)OR_BLOCK * d;
    memcpy(r->s16 + rec * (d / 32), sc + (int64_t)t * (d / 32) * 2, 2 * (size_t)(d / 32));
    return;
  }
  int nb = s->k_bits;
  int sl = or_slot(t);
  int64_t plane_words = (int64_t)(d / 32) * OR_BLOCK;
  if (s->k_codec == OR_POLAR_TREE) {
    const uint8_t* l1 = blk + 4 * (nb - 1) * plane_words;
    for (int a = 0; a < d; a++) {
      int c = 0;
      for (int p = 0; p < nb - 1; p++) {
        c |= or_getbit(blk, p * plane_words + (int64_t)(a / 32) * OR_BLOCK + sl, a % 32) << p;
      }
      if (a >= d / 2) {
        for (int x = 0; x < 2; x++) {
          c |= or_getbit(l1, x * (plane_words / 2) + (int64_t)((a - d / 2) / 32) * OR_BLOCK + sl, a % 32)
               << (nb - 1 + x);
        }
      }
      r->codes[rec * d + a] = (uint8_t)c;
    }
    memcpy(&r->n16[rec], l1 + 4 * plane_words + 2 * sl, 2);
    return;
  }
  for (int i = 0; i < d; i++) {
    int c = 0;
    for (int p = 0; p < nb; p++) {
      c |= or_getbit(blk, p * plane_words + (int64_t)(i / 32) * OR_BLOCK + sl, i % 32) << p;
    }
    r->codes[rec * d + i] = (uint8_t)c;
  }
  const uint8_t* after = blk + 4 * nb * plane_words;
  if (s->k_codec == OR_POLAR_QJL) {
    for (int j = 0; j < s->m; j++) {
      r->signs[rec * s->m + j] = (uint8_t)or_getbit(after, (int64_t)(j / 32) * OR_BLOCK + sl, j % 32);
    }
    after += 4 * (int64_t)(s->m / 32) * OR_BLOCK;
  }
  memcpy(&r->n16[rec], after + 2 * sl, 2);
  if (s->k_codec == OR_POLAR_QJL) memcpy(&r->rho16[rec], after + 2 * OR_BLOCK + 2 * sl, 2);
}

void or_pack_v(const or_spec* s, int b, int pos, int h, const or_vrec* r, int64_t rec, uint8_t* vc) {
  uint8_t* blk = or_vblock(s, b, pos, h, vc);
  int t = pos % OR_BLOCK;
  int d = s->d;
  if (s->v_codec == OR_RAW_F32) {
    memcpy(blk + (int64_t)t * d * 4, r->raw + rec * d, 4 * (size_t)d);
    return;
  }
  int nb = s->v_bits;
  int64_t plane_words = 4 * (int64_t)d;
  if (s->v_codec == OR_POLAR_TREE) {
    for (int p = 0; p < nb - 1; p++) {
      for (int a = 0; a < d; a++) {
        int bit = (r->codes[rec * d + a] >> p) & 1;
        or_setbit(blk, p * plane_words + (int64_t)(t / 32) * d + a, t % 32, bit);
      }
    }
    uint8_t* l1 = blk + 4 * (nb - 1) * plane_words;
    for (int x = 0; x < 2; x++) {
      for (int a = d / 2; a < d; a++) {
        int bit = (r->codes[rec * d + a] >> (nb - 1 + x)) & 1;
        or_setbit(l1, x * (plane_words / 2) + (int64_t)(t / 32) * (d / 2) + (a - d / 2), t % 32, bit);
      }
    }
    memcpy(l1 + 4 * plane_words + 2 * or_slot(t), &r->n16[rec], 2);
    return;
  }
  for (int p = 0; p < nb; p++) {
    for (int i = 0; i < d; i++) {
      int bit = (r->codes[rec * d + i] >> p) & 1;
      or_setbit(blk, p * plane_words + (int64_t)(t / 32) * d + i, t % 32, bit);
    }
  }
  memcpy(blk + 4 * nb * plane_words + 2 * or_slot(t), &r->n16[rec], 2);
}

void or_unpack_v(const or_spec* s, int b, int pos, int h, const uint8_t* vc, or_vrec* r, int64_t rec) {
  const uint8_t* blk = or_vblock(s, b, pos, h, (uint8_t*)vc);
  int t = pos % OR_BLOCK;
  int d = s->d;
  if (s->v_codec == OR_RAW_F32) {
    memcpy(r->raw + rec * d, blk + (int64_t)t * d * 4, 4 * (size_t)d);
    return;
  }
  int nb = s->v_bits;
  int64_t plane_words = 4 * (int64_t)d;
  if (s->v_codec == OR_POLAR_TREE) {
    const uint8_t* l1 = blk + 4 * (nb - 1) * plane_words;
    for (int a = 0; a < d; a++) {
      int c = 0;
      for (int p = 0; p < nb - 1; p++) {
        c |= or_getbit(blk, p * plane_words + (int64_t)(t / 32) * d + a, t % 32) << p;
      }
      if (a >= d / 2) {
        for (int x = 0; x < 2; x++) {
          c |= or_getbit(l1, x * (plane_words / 2) + (int64_t)(t / 32) * (d / 2) + (a - d / 2), t % 32)
               << (nb - 1 + x);
        }
      }
      r->codes[rec * d + a] = (uint8_t)c;
    }
    memcpy(&r->n16[rec], l1 + 4 * plane_words + 2 * or_slot(t), 2);
    return;
  }
  for (int i = 0; i < d; i++) {
    int c = 0;
    for (int p = 0; p < nb; p++) {
      c |= or_getbit(blk, p * plane_words + (int64_t)(t / 32) * d + i, t % 32) << p;
    }
    r->codes[rec * d + i] = (uint8_t)c;
  }
  memcpy(&r->n16[rec], blk + 4 * nb * plane_words + 2 * or_slot(t), 2);
}

/* ===================================================================== */
/* Many-vector quantise helpers                                          */
/* ===================================================================== */

void or_quantize_k_many(const or_spec* s, const float* DK, const uint16_t* c16,
                        const float* bounds, const float* S, int64_t n,
                        const float* x, or_krec* out, int64_t out_off) {
  int d = s->d;
  for (int64_t k = 0; k < n; k++) {
    const float* xv = x + k * d;
    int64_t rec = out_off + k;
    switch (s->k_codec) {
      case OR_RAW_F32:
        memcpy(out->raw + rec * d, xv, 4 * (size_t)d);
        break;
      case OR_Q8_BLOCK32:
        or_quantize_q8(xv, d, out->k8 + rec * d, out->s16 + rec * (d / 32), NULL);
        break;
      case OR_POLAR:
        or_quantize_polar(xv, d, s->k_bits, DK, c16, bounds, 0, NULL,
                          out->codes + rec * d, &out->n16[rec], NULL, NULL, NULL, NULL, NULL);
        break;
      case OR_POLAR_QJL:
        or_quantize_polar(xv, d, s->k_bits, DK, c16, bounds, s->m, S,
                          out->codes + rec * d, &out->n16[rec], out->signs + rec * s->m,
                          &out->rho16[rec], NULL, NULL, NULL);
        break;
      case OR_POLAR_TREE:
        or_quantize_tree(xv, d, DK, or_tree_table(s->k_bits), out->codes + rec * d, &out->n16[rec], NULL);
        break;
    }
  }
}

void or_quantize_v_many(const or_spec* s, const float* DV, const uint16_t* c16,
                        const float* bounds, int64_t n, const float* x,
                        or_vrec* out, int64_t out_off) {
  int d = s->d;
  for (int64_t k = 0; k < n; k++) {
    const float* xv = x + k * d;
    int64_t rec = out_off + k;
    if (s->v_codec == OR_RAW_F32) {
      memcpy(out->raw + rec * d, xv, 4 * (size_t)d);
    } else if (s->v_codec == OR_POLAR_TREE) {
      or_quantize_tree(xv, d, DV, or_tree_table(s->v_bits), out->codes + rec * d, &out->n16[rec], NULL);
    } else {
      or_quantize_polar(xv, d, s->v_bits, DV, c16, bounds, 0, NULL,
                        out->codes + rec * d, &out->n16[rec], NULL, NULL, NULL, NULL, NULL);
    }
  }
}

/* ===================================================================== */
/* Decode attention (fp64)                                               */
/* ===================================================================== */

static void or_dequant_k(const or_spec* s, const float* DK, const uint16_t* ck16,
                         const or_krec* kr, int64_t rec, double* out) {
  int d = s->d;
  switch (s->k_codec) {
    case OR_RAW_F32:
      for (int i = 0; i < d; i++) out[i] = (double)kr->raw[rec * d + i];
      break;
    case OR_Q8_BLOCK32:
      or_dequant_q8(d, kr->k8 + rec * d, kr->s16 + rec * (d / 32), out);
      break;
    case OR_POLAR_TREE:
      or_dequant_tree(d, DK, or_tree_table(s->k_bits), kr->codes + rec * d, kr->n16[rec], out);
      break;
    default:
      or_dequant_polar(d, DK, ck16, kr->codes + rec * d, kr->n16[rec], out);
      break;
  }
}

static void or_dequant_v(const or_spec* s, const float* DV, const uint16_t* cv16,
                         const or_vrec* vr, int64_t rec, double* out) {
  int d = s->d;
  if (s->v_codec == OR_RAW_F32) {
    for (int i = 0; i < d; i++) out[i] = (double)vr->raw[rec * d + i];
  } else if (s->v_codec == OR_POLAR_TREE) {
    or_dequant_tree(d, DV, or_tree_table(s->v_bits), vr->codes + rec * d, vr->n16[rec], out);
  } else {
    or_dequant_polar(d, DV, cv16, vr->codes + rec * d, vr->n16[rec], out);
  }
}

/* Reading: scale 1/sqrt(d), no mask, q head hq reads kv head hq / G.
 * For POLAR_QJL keys the logit is the QJL-corrected estimator of [P1]'s QJL paragraph:
 *   (<q, x_hat_t> + rho_t sqrt(pi/2)/m sum_j (S R q)_j sigma_tj) / sqrt(d),
 * with R q = H D_K q / sqrt(d) .  Softmax and the weighted sum of
 * dequantised values follow the textbook definition.  An empty sequence
 * yields a zero output. */
void or_decode_head(const or_spec* s, const float* DK, const float* DV, const uint16_t* ck16,
                    const uint16_t* cv16, const float* S, const or_krec* kr, const or_vrec* vr,
                    int b, int hq, int len, const float* q, double* out, double* logits_out) {
  int d = s->d;
  int G = s->n_q / s->n_kv;
  int h = hq / G;
  for (int i = 0; i < d; i++) out[i] = 0.0;
  if (len <= 0) return;
  double* sq = NULL;
  if (s->k_codec == OR_POLAR_QJL) {
    double* rq = (double*)malloc(sizeof(double) * d);
    for (int i = 0; i < d; i++) rq[i] = (double)DK[i] * (double)q[i];
    or_fwht_f64(rq, d);
    for (int i = 0; i < d; i++) rq[i] /= sqrt((double)d);
    sq = (double*)malloc(sizeof(double) * s->m);
    for (int j = 0; j < s->m; j++) {
      double acc = 0.0;
      for (int i = 0; i < d; i++) acc += (double)S[(size_t)j * d + i] * rq[i];
      sq[j] = acc;
    }
    free(rq);
  }
  double* lg = (double*)malloc(sizeof(double) * len);
  double* xh = (double*)malloc(sizeof(double) * d);
  double qjl_k = (s->k_codec == OR_POLAR_QJL) ? sqrt(M_PI / 2.0) / (double)s->m : 0.0;
  for (int t = 0; t < len; t++) {
    int64_t rec = ((int64_t)b * s->max_ctx + t) * s->n_kv + h;
    or_dequant_k(s, DK, ck16, kr, rec, xh);
    double dot = 0.0;
    for (int i = 0; i < d; i++) dot += (double)q[i] * xh[i];
    if (sq) {
      double sd = 0.0;
      for (int j = 0; j < s->m; j++) sd += sq[j] * (kr->signs[rec * s->m + j] ? 1.0 : -1.0);
      dot += (double)or_f16_to_f32(kr->rho16[rec]) * qjl_k * sd;
    }
    lg[t] = dot / sqrt((double)d);
    if (logits_out) logits_out[t] = lg[t];
  }
  double mx = lg[0];
  for (int t = 1; t < len; t++) if (lg[t] > mx) mx = lg[t];
  double den = 0.0;
  for (int t = 0; t < len; t++) { lg[t] = exp(lg[t] - mx); den += lg[t]; }
  for (int t = 0; t < len; t++) {
    int64_t rec = ((int64_t)b * s->max_ctx + t) * s->n_kv + h;
    or_dequant_v(s, DV, cv16, vr, rec, xh);
    double p = lg[t] / den;
    for (int i = 0; i < d; i++) out[i] += p * xh[i];
  }
  free(xh);
  free(lg);
  free(sq);
}

/* ===================================================================== */
/* Whole-cache helpers                                                   */
/* ===================================================================== */

void or_pack_cache(const or_spec* s, const int32_t* lens, const or_krec* kr, const or_vrec* vr,
                   uint8_t* kc, uint8_t* vc) {
  for (int b = 0; b < s->batch; b++) {
    for (int pos = 0; pos < lens[b]; pos++) {
      for (int h = 0; h < s->n_kv; h++) {
        int64_t rec = ((int64_t)b * s->max_ctx + pos) * s->n_kv + h;
        if (kc) or_pack_k(s, b, pos, h, kr, rec, kc);
        if (vc) or_pack_v(s, b, pos, h, vr, rec, vc);
      }
    }
  }
}

void or_unpack_cache(const or_spec* s, const int32_t* lens, const uint8_t* kc, const uint8_t* vc,
                     or_krec* kr, or_vrec* vr) {
  for (int b = 0; b < s->batch; b++) {
    for (int pos = 0; pos < lens[b]; pos++) {
      for (int h = 0; h < s->n_kv; h++) {
        int64_t rec = ((int64_t)b * s->max_ctx + pos) * s->n_kv + h;
        if (kc) or_unpack_k(s, b, pos, h, kc, kr, rec);
        if (vc) or_unpack_v(s, b, pos, h, vc, vr, rec);
      }
    }
  }
}

void or_decode_pairs(const or_spec* s, const float* DK, const float* DV, const uint16_t* ck16,
                     const uint16_t* cv16, const float* S, const or_krec* kr, const or_vrec* vr,
                     const int32_t* lens, const float* q, int n_pairs, const int32_t* pairs,
                     double* out, double* logits) {
  for (int k = 0; k < n_pairs; k++) {
    int b = pairs[2 * k];
    int hq = pairs[2 * k + 1];
    const float* qv = q + ((int64_t)b * s->n_q + hq) * s->d;
    or_decode_head(s, DK, DV, ck16, cv16, S, kr, vr, b, hq, lens[b], qv,
                   out + (int64_t)k * s->d, logits ? logits + (int64_t)k * s->max_ctx : NULL);
  }
}

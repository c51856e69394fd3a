/*
 * CPU oracle for blockwise-FP8 linear-layer GEMMs — TEST INFRASTRUCTURE ONLY.
 * Plain C; built with -O2 -ffp-contract=off and no fast-math so every float operation is
 * one IEEE binary32/binary64 operation rounded to nearest-even. OpenMP only splits
 * independent groups / output rows across threads; it changes no arithmetic.
 * Method statement: Paper walkthrough: Puro-2B (ta-paperlens.web.app), section
 * "Lever 2: use blockwise FP8 from step zero". See oracle.h for layouts and readings.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
static float f32_from(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* bfloat16 is the top half of an IEEE binary32: widening is exact. */
float oracle_bf16_to_f32(uint16_t h) { return f32_from((uint32_t)h << 16); }

/* OCP E4M3 ("fn") decode from the format definition: 1 sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinity. */
double oracle_e4m3_decode(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return sign ? -mag : mag;
}

/* Round |t| to the E4M3 grid with round-to-nearest, ties-to-even, by integer arithmetic on the
 * binary32 significand. Precondition: |t| <= 448 (callers clamp); larger inputs saturate to
 * the +-448 code. The sign is kept, so negative values that round to zero give 0x80. */
uint8_t oracle_e4m3_encode(float t) {
  uint32_t u = f32_bits(t);
  uint8_t sign = (uint8_t)((u >> 31) << 7);
  uint32_t a = u & 0x7fffffffu;
  int biased = (int)(a >> 23);
  if (biased == 0) return sign; /* zero or binary32 subnormal: far below 2^-10, rounds to 0 */
  if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7e); /* |t| >= 448: saturate */
  uint64_t sig = (uint64_t)((a & 0x7fffffu) | 0x800000u); /* |t| = sig * 2^(biased-150) */
  int e_t = biased - 127;                                  /* floor(log2 |t|) */
  int quantum = (e_t < -6 ? -6 : e_t) - 3; /* E4M3 spacing 2^quantum: 3 fraction bits, min normal 2^-6 */
  int shift = quantum - (biased - 150);    /* >= 20 */
  uint64_t q;
  if (shift >= 40) {
    q = 0;
  } else {
    uint64_t kept = sig >> shift;
    uint64_t rem = sig & ((1ull << shift) - 1);
    uint64_t half = 1ull << (shift - 1);
    q = kept;
    if (rem > half || (rem == half && (kept & 1))) q += 1;
  }
  /* |t| rounds to q * 2^quantum, with q in [0, 16]. */
  if (q == 0) return sign;
  if (q >= 16) { /* rounding carried into the next binade */
    q >>= 1;
    quantum += 1;
  }
  if (q < 8) return (uint8_t)(sign | q); /* subnormal: quantum is -9 here */
  int efield = quantum + 10;               /* value = (8+m) * 2^(efield-10) */
  uint32_t code = ((uint32_t)efield << 3) | (uint32_t)(q - 8);
  if (code > 0x7e) code = 0x7e;
  return (uint8_t)(sign | code);
}

void oracle_e4m3_encode_array(const float* t, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(t[i]);
}

/* Scale of one group from its max magnitude amax, and the factor that maps the group onto the
 * E4M3 range. Standard scales: s = amax/448 and r = 448/amax as single correctly-rounded binary32
 * divisions. Power-of-two scales (a variant of this library, not of the pages): s = 2^e for the
 * least integer e with 448 * 2^e >= amax, with e raised to -127 if it falls below (the least
 * power of two an 8-bit biased exponent holds); the payload is then x * 2^-e, exact. An all-zero
 * group has s = 1 in both modes. */
typedef struct {
  float scale;
  float recip; /* standard mode */
  int e;       /* power-of-two mode */
} group_scale_t;

static int pow2_exponent(float amax) {
  int e;
  (void)frexp((double)amax, &e); /* amax in [2^(e-1), 2^e) */
  e -= 9;                        /* a start near the answer; the two loops make it exact */
  while (ldexp(448.0, e) < (double)amax) ++e;
  while (ldexp(448.0, e - 1) >= (double)amax) --e;
  return e < -127 ? -127 : e;
}

static group_scale_t group_scale_of(float amax, int pow2) {
  group_scale_t g = {1.0f, 1.0f, 0};
  if (amax == 0.0f) return g;
  if (pow2) {
    g.e = pow2_exponent(amax);
    g.scale = (float)ldexp(1.0, g.e);
  } else {
    g.scale = amax / 448.0f;
    g.recip = 448.0f / amax;
  }
  return g;
}

/* The scaled value of one bf16 element, clamped to the E4M3 range, ready for encoding. */
static float scaled_value(uint16_t x, const group_scale_t* g, int pow2) {
  float t = pow2 ? (float)ldexp((double)oracle_bf16_to_f32(x), -g->e)
                 : oracle_bf16_to_f32(x) * g->recip;
  if (t > 448.0f) t = 448.0f;
  if (t < -448.0f) t = -448.0f;
  return t;
}

/* One quantisation group: `count` bf16 values at x[i*stride] -> q[i*qstride], scale *s.
 * amax = max |x|; scale as above; q = E4M3(clamp(x scaled, -448, 448)). */
void oracle_quant_group(const uint16_t* x, int64_t count, int64_t stride, uint8_t* q,
                        int64_t qstride, float* s, int pow2) {
  float amax = 0.0f;
  for (int64_t i = 0; i < count; ++i) {
    float v = fabsf(oracle_bf16_to_f32(x[i * stride]));
    if (v > amax) amax = v;
  }
  group_scale_t g = group_scale_of(amax, pow2);
  for (int64_t i = 0; i < count; ++i)
    q[i * qstride] = oracle_e4m3_encode(scaled_value(x[i * stride], &g, pow2));
  *s = g.scale;
}

/* Activations and their gradients: groups of 128 consecutive elements of a row (the row's
 * reduction dimension). Scale grid is chunk-major: s[c/128][r]. */
void oracle_quant_act_1x128(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q,
                            float* s, int pow2) {
  int64_t chunks = cols / 128;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < chunks; ++c)
      oracle_quant_group(x + r * cols + c * 128, 128, 1, q + r * cols + c * 128, 1,
                         s + c * rows + r, pow2);
}

/* Weights: one scale per 128x128 block, gathered row by row of the block. */
void oracle_quant_w_128x128(const uint16_t* w, int64_t n, int64_t k, uint8_t* q, float* s,
                            int pow2) {
  int64_t nb = n / 128, kb = k / 128;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb * kb; ++b) {
    int64_t bi = b / kb, bj = b % kb;
    float amax = 0.0f;
    for (int64_t i = 0; i < 128; ++i)
      for (int64_t j = 0; j < 128; ++j) {
        float v = fabsf(oracle_bf16_to_f32(w[(bi * 128 + i) * k + bj * 128 + j]));
        if (v > amax) amax = v;
      }
    group_scale_t g = group_scale_of(amax, pow2);
    for (int64_t i = 0; i < 128; ++i)
      for (int64_t j = 0; j < 128; ++j) {
        int64_t idx = (bi * 128 + i) * k + bj * 128 + j;
        q[idx] = oracle_e4m3_encode(scaled_value(w[idx], &g, pow2));
      }
    s[bi * kb + bj] = g.scale;
  }
}

/* Weight-gradient operands: the reduction dimension of dW = dY^T X is the token dimension,
 * so groups run down a column (128 consecutive rows). The result is stored transposed so that
 * each group is contiguous: qt[c][r], st[r/128][c]. Requantised from the bf16 source. */
void oracle_quant_transpose(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* qt,
                            float* st, int pow2) {
  int64_t chunks = rows / 128;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < cols; ++c)
    for (int64_t mb = 0; mb < chunks; ++mb)
      oracle_quant_group(x + mb * 128 * cols + c, 128, cols, qt + c * rows + mb * 128, 1,
                         st + mb * cols + c, pow2);
}

/* E4M3 values are integer multiples of 2^-9 with magnitude <= 448, so v*512 is an integer
 * (|.| <= 229376) and a 128-term dot product of such integers fits easily in int64: the chunk
 * product sum is exact. */
static int32_t dec512[256];
static int dec512_ready = 0;
static void init_dec512(void) {
  if (dec512_ready) return;
  for (int c = 0; c < 256; ++c) {
    double v = oracle_e4m3_decode((uint8_t)c);
    dec512[c] = isnan(v) ? 0 : (int32_t)(v * 512.0);
  }
  dec512_ready = 1;
}

/* Exact sum over one 128-chunk of a[i*as] * b[i*bs], returned as a double (exactly). */
static double chunk_dot(const uint8_t* a, int64_t as, const uint8_t* b, int64_t bs) {
  int64_t acc = 0;
  for (int64_t i = 0; i < 128; ++i) acc += (int64_t)dec512[a[i * as]] * dec512[b[i * bs]];
  return (double)acc / 262144.0; /* 2^18 */
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_gemm_fwd(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                     int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows,
                     double* out) {
  init_dec512();
  int64_t kbs = K / 128;
  if (!rows) nrows = M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ri = 0; ri < nrows; ++ri) {
    int64_t m = rows ? rows[ri] : ri;
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t kb = 0; kb < kbs; ++kb) {
        double p = chunk_dot(xq + m * K + kb * 128, 1, wq + n * K + kb * 128, 1);
        acc += (double)sx[kb * M + m] * (double)sw[(n / 128) * kbs + kb] * p;
      }
      out[ri * N + n] = acc;
    }
  }
}

void oracle_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw,
                       int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows,
                       double* out) {
  init_dec512();
  int64_t nbs = N / 128, kbs = K / 128;
  if (!rows) nrows = M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ri = 0; ri < nrows; ++ri) {
    int64_t m = rows ? rows[ri] : ri;
    for (int64_t k = 0; k < K; ++k) {
      double acc = 0.0;
      for (int64_t nb = 0; nb < nbs; ++nb) {
        double p = chunk_dot(dyq + m * N + nb * 128, 1, wq + nb * 128 * K + k, K);
        acc += (double)sdy[nb * M + m] * (double)sw[nb * kbs + k / 128] * p;
      }
      out[ri * K + k] = acc;
    }
  }
}

void oracle_gemm_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq,
                       const float* sxt, int64_t M, int64_t N, int64_t K, const int64_t* rows,
                       int64_t nrows, double* out) {
  init_dec512();
  int64_t mbs = M / 128;
  if (!rows) nrows = N;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ri = 0; ri < nrows; ++ri) {
    int64_t n = rows ? rows[ri] : ri;
    for (int64_t k = 0; k < K; ++k) {
      double acc = 0.0;
      for (int64_t mb = 0; mb < mbs; ++mb) {
        double p = chunk_dot(dytq + n * M + mb * 128, 1, xtq + k * M + mb * 128, 1);
        acc += (double)sdyt[mb * N + n] * (double)sxt[mb * K + k] * p;
      }
      out[ri * K + k] = acc;
    }
  }
}

/* ---------------------------------------------------------------- optimizer step
 * PuRo-2B news post (jj-blog-4lo.pages.dev), optimizer paragraph after the training-recipe
 * paragraph: the optimizer (Hyperball) updates the matrices that are roughly scale-invariant
 * and then scales each back to the Frobenius radius it had at initialisation, every step; the
 * other parameters use AdamW. (daker.ai page, five-choices section: the update is kept inside a
 * fixed radius.) The update direction of those matrices is not given on the pages; it is an
 * input here. Everything below is binary64 on binary32 inputs, returned unrounded. */

/* Frobenius norm sqrt(sum w_i^2); every square of a binary32 is exact in binary64. */
double oracle_frobenius_norm(const float* w, int64_t n) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += (double)w[i] * (double)w[i];
  return sqrt(ss);
}

/* One projected step: v = w - lr * u, then out = v * (radius / ||v||_F). A zero v is returned
 * unchanged (it has no direction to scale). */
void oracle_hyperball_update(const float* w, const float* u, int64_t n, double lr, double radius,
                             double* out) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double v = (double)w[i] - lr * (double)u[i];
    out[i] = v;
    ss += v * v;
  }
  double f = ss > 0.0 ? radius / sqrt(ss) : 1.0;
  for (int64_t i = 0; i < n; ++i) out[i] *= f;
}

/* AdamW with decoupled weight decay (Loshchilov and Hutter), step t >= 1:
 *   p <- p * (1 - lr * wd)
 *   m <- b1 * m + (1 - b1) * g          v <- b2 * v + (1 - b2) * g^2
 *   p <- p - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps) */
void oracle_adamw(const float* p, const float* g, const float* m, const float* v, int64_t n,
                  double lr, double b1, double b2, double eps, double wd, int64_t step,
                  double* p_out, double* m_out, double* v_out) {
  double c1 = 1.0 - pow(b1, (double)step), c2 = 1.0 - pow(b2, (double)step);
  for (int64_t i = 0; i < n; ++i) {
    double gi = (double)g[i];
    double mi = b1 * (double)m[i] + (1.0 - b1) * gi;
    double vi = b2 * (double)v[i] + (1.0 - b2) * gi * gi;
    double pi = (double)p[i] * (1.0 - lr * wd);
    pi -= lr * (mi / c1) / (sqrt(vi / c2) + eps);
    p_out[i] = pi;
    m_out[i] = mi;
    v_out[i] = vi;
  }
}

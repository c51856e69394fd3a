/*
 * CPU oracle for blockwise-FP8 linear-layer GEMMs — TEST INFRASTRUCTURE ONLY.
 *
 * This is the plain, slow, obviously-correct definition that the GPU library is checked
 * against. Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it. It shares no code, header, table or constant with the GPU library.
 *
 * What is computed, and where it is stated:
 *   Paper walkthrough: Puro-2B (ta-paperlens.web.app), section
 *   "Lever 2: use blockwise FP8 from step zero": only the linear-layer GEMMs run in FP8;
 *   one scale per local group — a 1x128 run along the GEMM's reduction dimension for
 *   activations and activation gradients, a 128x128 block for weights; masters stay BF16/FP32.
 *   PuRo-2B news post (jj-blog.pages.dev), driver-hack section, training-recipe paragraph:
 *   blockwise FP8 only for the linear-layer GEMMs, masters BF16/FP32, sequence 4096.
 *
 * Everything the pages leave open is a stated reading (listed in the repository's design
 * notes): OCP E4M3 ("fn": bias 7, max 448, no infinities, NaN = S.1111.111), scale
 * s = fl32(amax/448), payload q = E4M3_RNE(clamp(fl32(x * fl32(448/amax)), +-448)),
 * all-zero group -> s = 1, GEMM = sum over 128-chunks of sa*sb*(exact chunk dot product).
 *
 * Power-of-two scale variant (pow2 = 1; this library's option, not stated on the pages): a
 * nonzero group's scale is s = 2^e with e the least integer such that 448 * 2^e >= amax, raised
 * to -127 if it is smaller; the payload is q = E4M3_RNE(x * 2^-e), the product exact. Such
 * scales fit an 8-bit biased exponent (E8M0), which the matrix cores can apply themselves. The
 * GEMM definitions below are unchanged: they take whatever scales they are given.
 *
 * Layouts (all row-major, contiguous):
 *   bf16 tensors are passed as their raw uint16 bit patterns.
 *   quant_act_1x128 : x[rows][cols]          -> q[rows][cols], s[cols/128][rows]
 *   quant_w_128x128 : w[n][k]                -> q[n][k],       s[n/128][k/128]
 *   quant_transpose : x[rows][cols]          -> qt[cols][rows], st[rows/128][cols]
 *   gemm_fwd   : out[m][n] = sum_kb sx[kb][m]  * sw[n/128][kb] * sum_{k in kb} xq[m][k]*wq[n][k]
 *   gemm_dgrad : out[m][k] = sum_nb sdy[nb][m] * sw[nb][k/128] * sum_{n in nb} dyq[m][n]*wq[n][k]
 *   gemm_wgrad : out[n][k] = sum_mb sdyt[mb][n]* sxt[mb][k]    * sum_{m in mb} dytq[n][m]*xtq[k][m]
 * GEMM outputs are returned in double, unrounded. `rows`/`nrows` select a subset of output
 * rows (rows == NULL means all); out is then [nrows][cols_out].
 */
#ifndef BLOCKWISE_FP8_ORACLE_H
#define BLOCKWISE_FP8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

float oracle_bf16_to_f32(uint16_t h);
double oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e4m3_encode(float t);
void oracle_e4m3_encode_array(const float* t, int64_t n, uint8_t* out);
void oracle_quant_group(const uint16_t* x, int64_t count, int64_t stride, uint8_t* q,
                        int64_t qstride, float* s, int pow2);

void oracle_quant_act_1x128(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, float* s,
                            int pow2);
void oracle_quant_w_128x128(const uint16_t* w, int64_t n, int64_t k, uint8_t* q, float* s,
                            int pow2);
void oracle_quant_transpose(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* qt, float* st,
                            int pow2);

void oracle_gemm_fwd(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                     int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows,
                     double* out);
void oracle_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw,
                       int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows,
                       double* out);
void oracle_gemm_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq,
                       const float* sxt, int64_t M, int64_t N, int64_t K, const int64_t* rows,
                       int64_t nrows, double* out);
int oracle_num_threads(void);

/* Optimizer step (PuRo-2B news post, optimizer paragraph: scale-invariant matrices are scaled
 * back to their initial Frobenius radius every step; AdamW for the other parameters). binary64
 * arithmetic on binary32 inputs; results unrounded. */
double oracle_frobenius_norm(const float* w, int64_t n);
void oracle_hyperball_update(const float* w, const float* u, int64_t n, double lr, double radius,
                             double* out);
void oracle_adamw(const float* p, const float* g, const float* m, const float* v, int64_t n,
                  double lr, double b1, double b2, double eps, double wd, int64_t step,
                  double* p_out, double* m_out, double* v_out);

#ifdef __cplusplus
}
#endif
#endif

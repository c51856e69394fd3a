/*
 * puro.h — C ABI of libpuro.so: blockwise-FP8 quantisers and GEMMs for the linear layers of a
 * transformer, for AMD Instinct MI355X (gfx950).
 *
 * The operation (Paper walkthrough: Puro-2B, ta-paperlens.web.app, section
 * "Lever 2: use blockwise FP8 from step zero"; PuRo-2B news post, jj-blog.pages.dev,
 * driver-hack section, training-recipe paragraph): the linear-layer GEMMs — forward
 * Y = X·Wᵀ, data gradient dX = dY·W and weight gradient dW = dYᵀ·X — run on FP8 operands whose
 * scales are kept per local group: activations and activation gradients per 1x128 group along
 * the GEMM's reduction dimension, weights per 128x128 block. Masters stay in higher precision:
 * weights come in as bf16, Y and dX go out as bf16, dW goes out as fp32.
 *
 * Number formats fixed by this library where the pages are silent:
 *   payload  OCP FP8 E4M3 ("e4m3fn": bias 7, largest finite 448, no infinities,
 *            NaN = S.1111.111; never produced), one byte per element;
 *   scale    fp32 s = amax/448 (one correctly rounded division) for a group with max |x| = amax;
 *            an all-zero group has s = 1;
 *   payload  q = E4M3_RNE(clamp(x * (448/amax), -448, 448)) with 448/amax one correctly rounded
 *            fp32 division and the product one fp32 multiply; the sign of zero is kept;
 *   GEMM     out = sum over 128-element reduction chunks of (s_a * s_b) * (chunk dot product),
 *            the chunk dot product taken on matrix cores, the sum kept in fp32.
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE pointers owned by the caller; the library allocates, frees and
 *     synchronises nothing and keeps no state between calls (calls are thread-safe), except in
 *     debug mode (puro_set_debug below), where each call waits for its input checks.
 *   - Every tensor is dense row-major. Tensor pointers must be 16-byte aligned.
 *   - Every dimension must be a multiple of 128 (zero allowed). A call whose output is empty
 *     returns PURO_OK and launches nothing. A GEMM whose reduction dimension is 0 writes zeros
 *     (or leaves dW unchanged when accumulating).
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued asynchronously;
 *     the call returns once it is queued.
 *   - Validation is done on the host before anything is enqueued: a failed check returns a
 *     nonzero status and enqueues nothing. A failed launch returns PURO_ERR_LAUNCH.
 *   - Inputs must be finite, and a nonzero group must have amax >= 2^-119 (so that 448/amax is
 *     finite); such inputs are checked on the device only in debug mode.
 *   - Output buffers must not overlap inputs.
 */
#ifndef PURO_H
#define PURO_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PURO_OK = 0,
  PURO_ERR_NULL = 1,   /* a required pointer is NULL while its tensor is non-empty */
  PURO_ERR_SHAPE = 2,  /* a dimension is negative, not a multiple of 128, or too large */
  PURO_ERR_ALIGN = 3,  /* a tensor pointer is not 16-byte aligned */
  PURO_ERR_LAUNCH = 4, /* the HIP runtime rejected a kernel launch */
  PURO_ERR_ARG = 5,    /* another argument is out of range (e.g. `accumulate` not 0/1) */
  PURO_ERR_INPUT = 6   /* debug mode only: input data outside the contract (puro_set_debug) */
} puro_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char* puro_status_string(int status);
/* Version of this ABI; bumped on any incompatible change. */
int puro_abi_version(void);

/* 1x128 quantiser for activations (forward, groups along K) and activation gradients (dgrad,
 * groups along N): groups of 128 consecutive elements of each row.
 *   x  bf16 [rows][cols]        (input)
 *   q  e4m3 [rows][cols]        (output payload, same layout as x)
 *   s  fp32 [cols/128][rows]    (output scales, chunk-major: scales of one chunk column are
 *                                contiguous over rows) */
puro_status puro_quant_act_1x128(const void* x, int64_t rows, int64_t cols, void* q, float* s,
                                 void* stream);

/* 128x128 block quantiser for weights; one scale serves both the forward (reduce over K) and the
 * data-gradient GEMM (reduce over N) because the block is square.
 *   w  bf16 [n][k]              (input, the bf16 master copy)
 *   q  e4m3 [n][k]              (output payload)
 *   s  fp32 [n/128][k/128]      (output block scales) */
puro_status puro_quant_w_128x128(const void* w, int64_t n, int64_t k, void* q, float* s,
                                 void* stream);

/* Up to PURO_W_GROUP_MAX weight matrices quantised as puro_quant_w_128x128 in one launch (e.g.
 * every weight of a layer, whose bf16 masters all change at an optimiser step). Same outputs,
 * bit for bit, as one puro_quant_w_128x128 call per entry.
 *   items  host array of `count` entries (0 <= count <= PURO_W_GROUP_MAX), each with
 *          w bf16 [n][k], q e4m3 [n][k], s fp32 [n/128][k/128] as in puro_quant_w_128x128;
 *          entries with n or k = 0 are skipped
 * Every entry is validated before anything is enqueued; the first failure's status is
 * returned. count outside [0, PURO_W_GROUP_MAX] returns PURO_ERR_ARG. Outputs of different
 * entries must not overlap each other or any input. */
#define PURO_W_GROUP_MAX 8
typedef struct {
  const void* w;
  int64_t n, k;
  void* q;
  float* s;
} puro_w_item;
puro_status puro_quant_w_128x128_group(const puro_w_item* items, int count, void* stream);

/* Transposed 1x128 requantiser for the weight-gradient GEMM, whose reduction dimension is the
 * token dimension: groups of 128 consecutive ROWS of each column, requantised from bf16, and
 * written transposed so that every group is contiguous. Equals puro_quant_act_1x128 applied to
 * the transpose of x.
 *   x   bf16 [rows][cols]       (input, e.g. X[M][K] or dY[M][N])
 *   qt  e4m3 [cols][rows]       (output payload, transposed)
 *   st  fp32 [rows/128][cols]   (output scales) */
puro_status puro_quant_transpose(const void* x, int64_t rows, int64_t cols, void* qt, float* st,
                                 void* stream);

/* Both 1x128 orientations of one bf16 matrix from a single read of it: the row groups of
 * puro_quant_act_1x128 and the column groups of puro_quant_transpose, bit for bit the same
 * outputs as those two calls. The same passage defines both (1x128 runs along the reduction
 * dimension of the GEMM that consumes each copy): an activation X feeds the forward GEMM
 * (reduction over its columns) and the weight-gradient GEMM (reduction over its rows), and so
 * does an output gradient dY for the data-gradient and weight-gradient GEMMs.
 *   x   bf16 [rows][cols]       (input)
 *   q   e4m3 [rows][cols], s  fp32 [cols/128][rows]   (as puro_quant_act_1x128)
 *   qt  e4m3 [cols][rows], st fp32 [rows/128][cols]   (as puro_quant_transpose)
 * The four outputs must not overlap each other or x. */
puro_status puro_quant_dual_1x128(const void* x, int64_t rows, int64_t cols, void* q, float* s,
                                  void* qt, float* st, void* stream);

/* Forward GEMM  Y[m][n] = sum_kb sx[kb][m] * sw[n/128][kb] * sum_{k in kb} xq[m][k] * wq[n][k].
 *   xq e4m3 [M][K], sx fp32 [K/128][M]      (from puro_quant_act_1x128 of X)
 *   wq e4m3 [N][K], sw fp32 [N/128][K/128]  (from puro_quant_w_128x128 of W)
 *   y  bf16 [M][N]                           (output, round-to-nearest-even) */
puro_status puro_fp8_gemm_fwd(const void* xq, const float* sx, const void* wq, const float* sw,
                              void* y, int64_t M, int64_t N, int64_t K, void* stream);

/* Data-gradient GEMM  dX[m][k] = sum_nb sdy[nb][m] * sw[nb][k/128] * sum_{n in nb} dyq[m][n] * wq[n][k].
 * The weight payload and scales are the forward ones, used unchanged.
 *   dyq e4m3 [M][N], sdy fp32 [N/128][M]    (from puro_quant_act_1x128 of dY)
 *   wq  e4m3 [N][K], sw  fp32 [N/128][K/128]
 *   dx  bf16 [M][K]                          (output) */
puro_status puro_fp8_gemm_dgrad(const void* dyq, const float* sdy, const void* wq,
                                const float* sw, void* dx, int64_t M, int64_t N, int64_t K,
                                void* stream);

/* Weight-gradient GEMM  dW[n][k] (=, or += when accumulate = 1)
 *     sum_mb sdyt[mb][n] * sxt[mb][k] * sum_{m in mb} dytq[n][m] * xtq[k][m].
 *   dytq e4m3 [N][M], sdyt fp32 [M/128][N]  (from puro_quant_transpose of dY[M][N])
 *   xtq  e4m3 [K][M], sxt  fp32 [M/128][K]  (from puro_quant_transpose of X[M][K])
 *   dw   fp32 [N][K]                         (output; read too when accumulate = 1, which lets
 *                                             micro-batches sum into one FP32 gradient) */
puro_status puro_fp8_gemm_wgrad(const void* dytq, const float* sdyt, const void* xtq,
                                const float* sxt, float* dw, int64_t M, int64_t N, int64_t K,
                                int accumulate, void* stream);

/* Name of the kernel function puro_fp8_gemm_fwd (op 0), _dgrad (op 1) or _wgrad (op 2) -- or
 * its _pow2 twin when pow2 = 1 -- launches for the given sizes (e.g. "gemm_fwd_256x256"), as
 * the entry point itself chooses it on the current device; NULL when the call would launch
 * nothing or its arguments are invalid. For profiling and per-kernel accounting; static
 * storage, host only, enqueues nothing. */
const char* puro_gemm_kernel_name(int op, int64_t M, int64_t N, int64_t K, int pow2);

/* ---------------------------------------------------------------- optimizer step
 * PuRo-2B news post (jj-blog-4lo.pages.dev), optimizer paragraph after the training-recipe
 * paragraph: the roughly scale-invariant matrices (the linear-layer weights) are updated and
 * then scaled back to the Frobenius radius they had at initialisation, every step; the other
 * parameters use AdamW. The pages do not give the matrices' update direction (their MuonH
 * orthogonalisation), so the projected step takes it as an input. Masters are fp32; the
 * projected step also writes the bf16 copy that puro_quant_w_128x128 reads next.
 *
 * Conventions as above, plus: numel must be a multiple of 4 (PURO_ERR_SHAPE otherwise);
 * `workspace` is caller-owned device memory of at least PURO_OPT_WORKSPACE_BYTES bytes,
 * 16-byte aligned, used by one call at a time (calls sharing a workspace must be ordered on
 * one stream). Reductions run in a fixed order set by numel alone, so results repeat exactly. */
#define PURO_OPT_MAX_BLOCKS 2048
#define PURO_OPT_WORKSPACE_BYTES (8 * PURO_OPT_MAX_BLOCKS + 256)

/* Frobenius norm of w (fp32 [numel]), summed in fp64, written as fp32 to the device float
 * *norm (e.g. a matrix's radius at initialisation). */
puro_status puro_frobenius_norm(const float* w, int64_t numel, float* norm, void* workspace,
                                void* stream);

/* Projected step of one matrix, in place:
 *   v = w - lr * u            (one fused multiply-add per element, fp32)
 *   w = v * (radius / ||v||_F) (||v|| summed in fp64; the factor rounded once to fp32;
 *                               a zero v is left unchanged)
 *   w_bf16 = bf16_rne(w)
 *   w       fp32 [numel], updated in place;  u fp32 [numel], the update direction
 *   radius  DEVICE pointer to one fp32 (e.g. from puro_frobenius_norm at initialisation), so a
 *           whole optimizer step can be captured without host round trips
 *   w_bf16  bf16 [numel] (output) */
puro_status puro_hyperball_step(float* w, const float* u, int64_t numel, float lr,
                                const float* radius, void* w_bf16, void* workspace,
                                void* stream);

/* puro_hyperball_step without the workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the partial sums go to a scratch array the library keeps in device memory,
 * PURO_OPT_WORKSPACE_BYTES per device, held until the process ends. Its need does not depend on
 * numel, so every numel that puro_hyperball_step accepts fits (larger numel: PURO_ERR_SHAPE).
 * Same arguments otherwise, same validation, same kernels and the same results bit for bit.
 * The call allocates and frees nothing. The first call on a device looks up the array's
 * address there (PURO_ERR_LAUNCH if that fails). All calls on one device share the array:
 * calls that overlap in time on one device (different streams, no ordering between them) race
 * and give wrong results; order them on one stream. */
puro_status puro_hyperball_step_noalloc(float* w, const float* u, int64_t numel, float lr,
                                        const float* radius, void* w_bf16, void* stream);

/* AdamW with decoupled weight decay (Loshchilov and Hutter), in place on fp32 state:
 *   m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*g^2
 *   p = p*(1 - lr*wd) - lr * (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps)
 * p, g, m, v fp32 [numel]; p_bf16 (optional, NULL to skip) bf16 [numel] receives bf16_rne(p).
 * hp is a host struct; step t >= 1, 0 <= beta < 1 and eps > 0, else PURO_ERR_ARG. */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  int64_t step;
} puro_adamw_params;
puro_status puro_adamw_step(float* p, const float* g, float* m, float* v, int64_t numel,
                            const puro_adamw_params* hp, void* p_bf16, void* stream);

/* ---------------------------------------------------------------- power-of-two scales
 * A variant of every entry point above with the same arguments, layouts and validation, whose
 * scales are powers of two. This is an option of this library, not the pages' rule; the
 * grouping (1x128 along the reduction dimension, 128x128 weight blocks) is theirs, as above.
 *   scale    s = 2^e for the least integer e with 448 * 2^e >= amax, raised to -127 when it is
 *            smaller (so tiny groups need no lower bound on amax); an all-zero group has s = 1;
 *            s is stored as an ordinary fp32 value (2^-127 as the fp32 subnormal 0x00400000);
 *   payload  q = E4M3_RNE(x * 2^-e), the product exact; |x * 2^-e| <= 448 needs no clamp;
 *   GEMM     the same sums as above, with each operand's scale applied by the matrix cores as an
 *            8-bit biased exponent (E8M0) and the chunk results accumulated by them in fp32.
 * The _pow2 GEMMs read only the exponent field (bits 23-30) of each scale: they are meant for
 * scales from the _pow2 quantisers, and take any other positive scale s as 2^floor(log2 s).
 * Compared with amax/448 scales, a group's largest magnitude maps into (224, 448] instead of
 * exactly onto 448: normal payloads keep their 3 mantissa bits, but up to one binade of E4M3
 * range goes unused at the top, so small elements reach the subnormal range up to 2x sooner and
 * amax itself is rounded like any other element. In exchange the GEMMs do no fp32 promotion
 * work outside the matrix cores. */
puro_status puro_quant_act_1x128_pow2(const void* x, int64_t rows, int64_t cols, void* q, float* s,
                                      void* stream);
puro_status puro_quant_w_128x128_pow2(const void* w, int64_t n, int64_t k, void* q, float* s,
                                      void* stream);
puro_status puro_quant_w_128x128_group_pow2(const puro_w_item* items, int count, void* stream);
puro_status puro_quant_transpose_pow2(const void* x, int64_t rows, int64_t cols, void* qt,
                                      float* st, void* stream);
puro_status puro_quant_dual_1x128_pow2(const void* x, int64_t rows, int64_t cols, void* q,
                                       float* s, void* qt, float* st, void* stream);
puro_status puro_fp8_gemm_fwd_pow2(const void* xq, const float* sx, const void* wq,
                                   const float* sw, void* y, int64_t M, int64_t N, int64_t K,
                                   void* stream);
puro_status puro_fp8_gemm_dgrad_pow2(const void* dyq, const float* sdy, const void* wq,
                                     const float* sw, void* dx, int64_t M, int64_t N, int64_t K,
                                     void* stream);
puro_status puro_fp8_gemm_wgrad_pow2(const void* dytq, const float* sdyt, const void* xtq,
                                     const float* sxt, float* dw, int64_t M, int64_t N, int64_t K,
                                     int accumulate, void* stream);

/* Debug mode: input checks on the device before every quantiser and GEMM.
 * At level 0 (the default) nothing is checked. At level 1 or more each quantiser and GEMM
 * entry point, after its host validation, scans its inputs on `stream`, waits for the scan
 * (the call then synchronises the stream, so debug mode is not for graph capture) and returns
 * PURO_ERR_INPUT, enqueueing nothing more, when they break the contract above:
 *   - quantisers: a bf16 NaN or infinity; with the amax/448 rule (not the _pow2 one, which has
 *     no lower bound) a group of the entry point's shape whose amax is nonzero and below 2^-119;
 *   - GEMMs: an E4M3 NaN code (0x7F or 0xFF) in either operand, or a scale that is not a
 *     positive finite float.
 * The level starts from the environment variable PURO_DEBUG (a positive integer; unset or 0
 * means off), read the first time it is needed; puro_set_debug overrides it for the process
 * (negative values mean 0). Checks are serialised by the library; the scans are plain and slow,
 * meant for finding bad data, not for production runs. */
void puro_set_debug(int level);
int puro_debug_level(void);

#ifdef __cplusplus
}
#endif
#endif /* PURO_H */

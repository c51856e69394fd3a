// Blockwise FP8 quantisers for gfx950: 1x128 row groups, 128x128 weight blocks (one matrix or
// several in one launch), the transposed 1x128 requantisation used by the weight-gradient GEMM,
// and both 1x128 orientations from one read.
//
// Method: Paper walkthrough: Puro-2B (ta-paperlens.web.app), section "Lever 2: use blockwise
// FP8 from step zero" — one fp32 scale per local group: a 1x128 run along the consuming GEMM's
// reduction dimension for activations and activation gradients, a 128x128 block for weights.
// Number formats and rounding as stated in include/puro.h. Every kernel is instantiated for two
// scale rules: amax/448 (the reading of the pages) and the power of two at or above it (a
// library option).
//
// All of them are HBM-bound: each bf16 element is read once (2 B) and each of its E4M3 codes
// written once (1 B per copy), plus one fp32 scale per group. Loads are 16 B per lane and every
// wave instruction touches whole 128 B (or larger) segments; all per-element arithmetic (widen,
// |max|, multiply, clamp, packed convert) stays in registers.
#include "common.hpp"
#include "debug.hpp"

namespace puro {
namespace {

// 16 bytes of an input each quantiser reads exactly once, loaded non-temporally so that the
// bf16 source does not displace, in L2 and the memory-side cache, the e4m3 copies the GEMMs
// read next. Measured on the model step: the quantisers and the following data gradient got
// faster, the step 2.2 % (the dual quantiser alone with plain loads elsewhere made the weight
// quantiser slower; every quantiser together is what pays).
__device__ __forceinline__ uint4 load_once16(const uint16_t* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  uint4 v;
  v.x = t[0];
  v.y = t[1];
  v.z = t[2];
  v.w = t[3];
  return v;
}

// ------------------------------------------------------------------ 1x128 row groups
// One group = 128 consecutive bf16 of a row = 16 lanes x 8 elements. A 256-thread block holds
// 16 groups per pass and makes 4 passes, so it covers 64 consecutive rows of one 128-column
// chunk. Blocks walk the chunks of a row band first so neighbouring blocks read neighbouring
// 256 B segments of the same rows.
constexpr int kActPasses = 4;
constexpr int kActRowsPerBlock = 16 * kActPasses;

template <bool kPow2>
__global__ __launch_bounds__(256) void quant_act_1x128_kernel(const uint16_t* __restrict__ x,
                                                              int64_t rows, int64_t cols,
                                                              uint8_t* __restrict__ q,
                                                              float* __restrict__ s) {
  const int64_t chunks = cols >> 7;
  const int64_t c = blockIdx.x % chunks;
  const int64_t rb = blockIdx.x / chunks;
  const int seg = threadIdx.x >> 4;
  const int l16 = threadIdx.x & 15;

  uint4 v[kActPasses];
#pragma unroll
  for (int p = 0; p < kActPasses; ++p) {
    const int64_t row = rb * kActRowsPerBlock + p * 16 + seg;
    v[p] = load_once16(x + row * cols + c * 128 + l16 * 8);
  }
#pragma unroll
  for (int p = 0; p < kActPasses; ++p) {
    const int64_t row = rb * kActRowsPerBlock + p * 16 + seg;
    float f[8] = {bf16_lo(v[p].x), bf16_hi(v[p].x), bf16_lo(v[p].y), bf16_hi(v[p].y),
                  bf16_lo(v[p].z), bf16_hi(v[p].z), bf16_lo(v[p].w), bf16_hi(v[p].w)};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, __builtin_fabsf(f[i]));
    m = row16_max(m);
    float sc, r;
    scale_rule<kPow2>(m, sc, r);
    uint2 out;
    out.x = e4m3x4(f[0] * r, f[1] * r, f[2] * r, f[3] * r);
    out.y = e4m3x4(f[4] * r, f[5] * r, f[6] * r, f[7] * r);
    *reinterpret_cast<uint2*>(q + row * cols + c * 128 + l16 * 8) = out;
    if (l16 == 0) s[c * rows + row] = sc;
  }
}

// ------------------------------------------------------------------ 128x128 weight blocks
// One 256-thread block per 128x128 block: 16 lanes cover a 256 B row, 8 passes of 16 rows.
template <bool kPow2>
__device__ __forceinline__ void quant_w_block(const uint16_t* __restrict__ w, int64_t n, int64_t k,
                                              uint8_t* __restrict__ q, float* __restrict__ s,
                                              int64_t blk, float* wave_max) {
  const int64_t kblocks = k >> 7;
  const int64_t bj = blk % kblocks;
  const int64_t bi = blk / kblocks;
  const int t = threadIdx.x;
  const int r0 = t >> 4;
  const int col = (t & 15) * 8;

  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = bi * 128 + r0 + 16 * i;
    v[i] = load_once16(w + row * k + bj * 128 + col);
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m = fmaxf(m, __builtin_fabsf(bf16_lo(v[i].x)));
    m = fmaxf(m, __builtin_fabsf(bf16_hi(v[i].x)));
    m = fmaxf(m, __builtin_fabsf(bf16_lo(v[i].y)));
    m = fmaxf(m, __builtin_fabsf(bf16_hi(v[i].y)));
    m = fmaxf(m, __builtin_fabsf(bf16_lo(v[i].z)));
    m = fmaxf(m, __builtin_fabsf(bf16_hi(v[i].z)));
    m = fmaxf(m, __builtin_fabsf(bf16_lo(v[i].w)));
    m = fmaxf(m, __builtin_fabsf(bf16_hi(v[i].w)));
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((t & 63) == 0) wave_max[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  float sc, r;
  scale_rule<kPow2>(m, sc, r);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = bi * 128 + r0 + 16 * i;
    uint2 out;
    out.x = e4m3x4(bf16_lo(v[i].x) * r, bf16_hi(v[i].x) * r, bf16_lo(v[i].y) * r,
                   bf16_hi(v[i].y) * r);
    out.y = e4m3x4(bf16_lo(v[i].z) * r, bf16_hi(v[i].z) * r, bf16_lo(v[i].w) * r,
                   bf16_hi(v[i].w) * r);
    *reinterpret_cast<uint2*>(q + row * k + bj * 128 + col) = out;
  }
  if (t == 0) s[bi * kblocks + bj] = sc;
}

template <bool kPow2>
__global__ __launch_bounds__(256) void quant_w_128x128_kernel(const uint16_t* __restrict__ w,
                                                              int64_t n, int64_t k,
                                                              uint8_t* __restrict__ q,
                                                              float* __restrict__ s) {
  __shared__ float wave_max[4];
  quant_w_block<kPow2>(w, n, k, q, s, blockIdx.x, wave_max);
}

// Several weight matrices in one launch: block b belongs to the entry whose range of block
// indices [first[i], first[i+1]) holds it.
constexpr int kWGroupMax = PURO_W_GROUP_MAX;
struct WGroup {
  const uint16_t* w[kWGroupMax];
  uint8_t* q[kWGroupMax];
  float* s[kWGroupMax];
  int64_t n[kWGroupMax], k[kWGroupMax];
  int64_t first[kWGroupMax + 1];
  int count;
};

template <bool kPow2>
__global__ __launch_bounds__(256) void quant_w_128x128_group_kernel(const WGroup g) {
  __shared__ float wave_max[4];
  const int64_t b = blockIdx.x;
  int i = 0;
  while (i + 1 < g.count && b >= g.first[i + 1]) ++i;
  quant_w_block<kPow2>(g.w[i], g.n[i], g.k[i], g.q[i], g.s[i], b - g.first[i], wave_max);
}

// ------------------------------------------------------------------ column groups, and both at once
// One 512-thread block per 128x128 tile of x, read from HBM once. Pass 1: 16 lanes per 256 B
// row, 4 passes of 32 rows; the tile is staged in LDS as dwords with a 65-dword row pitch and,
// with kRows, each row's 128 values also form one row group, quantised and stored from
// registers. Pass 2: 8 lanes per column pair, each holding 16 rows, so a column's amax is an
// 8-lane reduction and its 128 output bytes (the transposed copy) are one contiguous 128 B
// segment; the 8 waves cover the 64 column pairs in one round. (Eight waves per block rather
// than four: twice the waves per CU for the same 33 KB of LDS, measured 2 % faster over the
// model's shapes.) Without kRows this is the transposed quantiser on its own: it replaced a
// 128x64-tile kernel whose 128 B row segments read HBM less efficiently.
constexpr int kDualPitch = 65;  // dwords per staged row (64 data + 1 pad)

template <bool kPow2, bool kRows>
__global__ __launch_bounds__(512) void quant_dual_1x128_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, uint8_t* __restrict__ q,
    float* __restrict__ s, uint8_t* __restrict__ qt, float* __restrict__ st) {
  __shared__ uint32_t tile[128 * kDualPitch];
  const int64_t cblocks = cols >> 7;
  const int64_t cb = blockIdx.x % cblocks;
  const int64_t mb = blockIdx.x / cblocks;
  const int64_t m0 = mb * 128, c0 = cb * 128;
  const int t = threadIdx.x;

  {
    const int seg = t >> 4, l16 = t & 15;
    uint4 v[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      v[p] = load_once16(x + (m0 + 32 * p + seg) * cols + c0 + l16 * 8);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = 32 * p + seg;
      uint32_t* dst = tile + r * kDualPitch + l16 * 4;
      dst[0] = v[p].x;
      dst[1] = v[p].y;
      dst[2] = v[p].z;
      dst[3] = v[p].w;
      if constexpr (!kRows) continue;
      const float f[8] = {bf16_lo(v[p].x), bf16_hi(v[p].x), bf16_lo(v[p].y), bf16_hi(v[p].y),
                          bf16_lo(v[p].z), bf16_hi(v[p].z), bf16_lo(v[p].w), bf16_hi(v[p].w)};
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, __builtin_fabsf(f[i]));
      m = row16_max(m);
      float sc, rc;
      scale_rule<kPow2>(m, sc, rc);
      uint2 out;
      out.x = e4m3x4(f[0] * rc, f[1] * rc, f[2] * rc, f[3] * rc);
      out.y = e4m3x4(f[4] * rc, f[5] * rc, f[6] * rc, f[7] * rc);
      *reinterpret_cast<uint2*>(q + (m0 + r) * cols + c0 + l16 * 8) = out;
      if (l16 == 0) s[cb * rows + m0 + r] = sc;
    }
  }
  __syncthreads();

  const int lane = t & 63, w = t >> 6;
  const int pair = lane & 7, g = lane >> 3;
  {
    const int dc = w * 8 + pair;  // dword column: tile columns 2*dc, 2*dc+1
    // Lanes of groups g and g + 4 would hit the same LDS banks row for row (16 rows x 65
    // dwords apart = 16 banks, mod 64); the upper four groups therefore walk their 16 rows
    // starting at row 8, so every read instruction touches 64 distinct banks. d[i] holds row
    // 16g + ((i + rot) mod 16), and the encoded halves are swapped back below.
    const int rot = (g >> 2) << 3;
    const uint32_t* grp = tile + 16 * g * kDualPitch + dc;
    const uint32_t* lo = grp + rot * kDualPitch;        // rows rot .. rot + 7
    const uint32_t* hi = grp + (8 - rot) * kDualPitch;  // the other 8 rows
    uint32_t d[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      d[i] = lo[i * kDualPitch];
      d[8 + i] = hi[i * kDualPitch];
    }
    float m0v = 0.0f, m1v = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      m0v = fmaxf(m0v, __builtin_fabsf(bf16_lo(d[i])));
      m1v = fmaxf(m1v, __builtin_fabsf(bf16_hi(d[i])));
    }
    m0v = stride8_max(m0v);
    m1v = stride8_max(m1v);
    float s0, r0, s1, r1;
    scale_rule<kPow2>(m0v, s0, r0);
    scale_rule<kPow2>(m1v, s1, r1);
    uint4 o0, o1;
    o0.x = e4m3x4(bf16_lo(d[0]) * r0, bf16_lo(d[1]) * r0, bf16_lo(d[2]) * r0, bf16_lo(d[3]) * r0);
    o0.y = e4m3x4(bf16_lo(d[4]) * r0, bf16_lo(d[5]) * r0, bf16_lo(d[6]) * r0, bf16_lo(d[7]) * r0);
    o0.z = e4m3x4(bf16_lo(d[8]) * r0, bf16_lo(d[9]) * r0, bf16_lo(d[10]) * r0, bf16_lo(d[11]) * r0);
    o0.w = e4m3x4(bf16_lo(d[12]) * r0, bf16_lo(d[13]) * r0, bf16_lo(d[14]) * r0, bf16_lo(d[15]) * r0);
    o1.x = e4m3x4(bf16_hi(d[0]) * r1, bf16_hi(d[1]) * r1, bf16_hi(d[2]) * r1, bf16_hi(d[3]) * r1);
    o1.y = e4m3x4(bf16_hi(d[4]) * r1, bf16_hi(d[5]) * r1, bf16_hi(d[6]) * r1, bf16_hi(d[7]) * r1);
    o1.z = e4m3x4(bf16_hi(d[8]) * r1, bf16_hi(d[9]) * r1, bf16_hi(d[10]) * r1, bf16_hi(d[11]) * r1);
    o1.w = e4m3x4(bf16_hi(d[12]) * r1, bf16_hi(d[13]) * r1, bf16_hi(d[14]) * r1, bf16_hi(d[15]) * r1);
    if (rot) {  // back to row order: rows 0-7 of the group are in the upper eight bytes
      o0 = make_uint4(o0.z, o0.w, o0.x, o0.y);
      o1 = make_uint4(o1.z, o1.w, o1.x, o1.y);
    }
    const int64_t col = c0 + 2 * dc;
    *reinterpret_cast<uint4*>(qt + col * rows + m0 + 16 * g) = o0;
    *reinterpret_cast<uint4*>(qt + (col + 1) * rows + m0 + 16 * g) = o1;
    if (g == 0) *reinterpret_cast<float2*>(st + mb * cols + col) = make_float2(s0, s1);
  }
}

// ------------------------------------------------------------------ host side
// Each entry point validates its arguments on the host, then launches the kernel instantiated
// for its scale rule (amax/448, or the power of two at or above it).
template <bool kPow2>
puro_status quant_act_1x128(const void* x, int64_t rows, int64_t cols, void* q, float* s,
                            void* stream) {
  if (!dim_ok(rows) || !dim_ok(cols)) return PURO_ERR_SHAPE;
  const bool empty = rows == 0 || cols == 0;
  PURO_TRY(check_ptr(x, empty));
  PURO_TRY(check_ptr(q, empty));
  PURO_TRY(check_ptr(s, empty));
  if (empty) return PURO_OK;
  PURO_TRY(debug::check_bf16(x, rows, cols, debug::kRowGroups, kPow2, stream));
  const int64_t blocks = (rows / kActRowsPerBlock) * (cols / 128);
  if (blocks > INT32_MAX) return PURO_ERR_SHAPE;
  hipLaunchKernelGGL(quant_act_1x128_kernel<kPow2>, dim3(static_cast<uint32_t>(blocks)),
                     dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(x), rows, cols, static_cast<uint8_t*>(q), s);
  return launch_status();
}

template <bool kPow2>
puro_status quant_w_128x128(const void* w, int64_t n, int64_t k, void* q, float* s,
                            void* stream) {
  if (!dim_ok(n) || !dim_ok(k)) return PURO_ERR_SHAPE;
  const bool empty = n == 0 || k == 0;
  PURO_TRY(check_ptr(w, empty));
  PURO_TRY(check_ptr(q, empty));
  PURO_TRY(check_ptr(s, empty));
  if (empty) return PURO_OK;
  PURO_TRY(debug::check_bf16(w, n, k, debug::kBlockGroups, kPow2, stream));
  const int64_t blocks = (n / 128) * (k / 128);
  if (blocks > INT32_MAX) return PURO_ERR_SHAPE;
  hipLaunchKernelGGL(quant_w_128x128_kernel<kPow2>, dim3(static_cast<uint32_t>(blocks)),
                     dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(w), n, k, static_cast<uint8_t*>(q), s);
  return launch_status();
}

template <bool kPow2>
puro_status quant_transpose(const void* x, int64_t rows, int64_t cols, void* qt, float* st,
                            void* stream) {
  if (!dim_ok(rows) || !dim_ok(cols)) return PURO_ERR_SHAPE;
  const bool empty = rows == 0 || cols == 0;
  PURO_TRY(check_ptr(x, empty));
  PURO_TRY(check_ptr(qt, empty));
  PURO_TRY(check_ptr(st, empty));
  if (empty) return PURO_OK;
  PURO_TRY(debug::check_bf16(x, rows, cols, debug::kColGroups, kPow2, stream));
  const int64_t blocks = (rows / 128) * (cols / 128);
  if (blocks > INT32_MAX) return PURO_ERR_SHAPE;
  const auto kernel = quant_dual_1x128_kernel<kPow2, false>;  // column groups only
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(512), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(x), rows, cols, nullptr, nullptr,
                     static_cast<uint8_t*>(qt), st);
  return launch_status();
}

template <bool kPow2>
puro_status quant_dual_1x128(const void* x, int64_t rows, int64_t cols, void* q, float* s,
                             void* qt, float* st, void* stream) {
  if (!dim_ok(rows) || !dim_ok(cols)) return PURO_ERR_SHAPE;
  const bool empty = rows == 0 || cols == 0;
  PURO_TRY(check_ptr(x, empty));
  PURO_TRY(check_ptr(q, empty));
  PURO_TRY(check_ptr(s, empty));
  PURO_TRY(check_ptr(qt, empty));
  PURO_TRY(check_ptr(st, empty));
  if (empty) return PURO_OK;
  PURO_TRY(debug::check_bf16(x, rows, cols, debug::kRowGroups | debug::kColGroups, kPow2,
                             stream));
  const int64_t blocks = (rows / 128) * (cols / 128);
  if (blocks > INT32_MAX) return PURO_ERR_SHAPE;
  const auto kernel = quant_dual_1x128_kernel<kPow2, true>;
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(512), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(x), rows, cols, static_cast<uint8_t*>(q), s,
                     static_cast<uint8_t*>(qt), st);
  return launch_status();
}

template <bool kPow2>
puro_status quant_w_128x128_group(const puro_w_item* items, int count, void* stream) {
  if (count < 0 || count > kWGroupMax) return PURO_ERR_ARG;
  if (count == 0) return PURO_OK;
  if (items == nullptr) return PURO_ERR_NULL;
  WGroup g = {};
  int64_t blocks = 0;
  int used = 0;
  for (int i = 0; i < count; ++i) {
    const puro_w_item& it = items[i];
    if (!dim_ok(it.n) || !dim_ok(it.k)) return PURO_ERR_SHAPE;
    const bool empty = it.n == 0 || it.k == 0;
    PURO_TRY(check_ptr(it.w, empty));
    PURO_TRY(check_ptr(it.q, empty));
    PURO_TRY(check_ptr(it.s, empty));
    if (empty) continue;
    g.w[used] = static_cast<const uint16_t*>(it.w);
    g.q[used] = static_cast<uint8_t*>(it.q);
    g.s[used] = it.s;
    g.n[used] = it.n;
    g.k[used] = it.k;
    g.first[used] = blocks;
    blocks += (it.n / 128) * (it.k / 128);
    ++used;
  }
  if (used == 0) return PURO_OK;
  if (blocks > INT32_MAX) return PURO_ERR_SHAPE;
  for (int i = 0; i < used; ++i)
    PURO_TRY(debug::check_bf16(g.w[i], g.n[i], g.k[i], debug::kBlockGroups, kPow2, stream));
  g.first[used] = blocks;
  g.count = used;
  hipLaunchKernelGGL(quant_w_128x128_group_kernel<kPow2>, dim3(static_cast<uint32_t>(blocks)),
                     dim3(256), 0, static_cast<hipStream_t>(stream), g);
  return launch_status();
}

}  // namespace
}  // namespace puro

using namespace puro;

extern "C" puro_status puro_quant_act_1x128(const void* x, int64_t rows, int64_t cols, void* q,
                                            float* s, void* stream) {
  return quant_act_1x128<false>(x, rows, cols, q, s, stream);
}
extern "C" puro_status puro_quant_w_128x128(const void* w, int64_t n, int64_t k, void* q,
                                            float* s, void* stream) {
  return quant_w_128x128<false>(w, n, k, q, s, stream);
}
extern "C" puro_status puro_quant_transpose(const void* x, int64_t rows, int64_t cols, void* qt,
                                            float* st, void* stream) {
  return quant_transpose<false>(x, rows, cols, qt, st, stream);
}
extern "C" puro_status puro_quant_dual_1x128(const void* x, int64_t rows, int64_t cols, void* q,
                                             float* s, void* qt, float* st, void* stream) {
  return quant_dual_1x128<false>(x, rows, cols, q, s, qt, st, stream);
}
extern "C" puro_status puro_quant_w_128x128_group(const puro_w_item* items, int count,
                                                  void* stream) {
  return quant_w_128x128_group<false>(items, count, stream);
}

extern "C" puro_status puro_quant_act_1x128_pow2(const void* x, int64_t rows, int64_t cols,
                                                 void* q, float* s, void* stream) {
  return quant_act_1x128<true>(x, rows, cols, q, s, stream);
}
extern "C" puro_status puro_quant_w_128x128_pow2(const void* w, int64_t n, int64_t k, void* q,
                                                 float* s, void* stream) {
  return quant_w_128x128<true>(w, n, k, q, s, stream);
}
extern "C" puro_status puro_quant_transpose_pow2(const void* x, int64_t rows, int64_t cols,
                                                 void* qt, float* st, void* stream) {
  return quant_transpose<true>(x, rows, cols, qt, st, stream);
}
extern "C" puro_status puro_quant_dual_1x128_pow2(const void* x, int64_t rows, int64_t cols,
                                                  void* q, float* s, void* qt, float* st,
                                                  void* stream) {
  return quant_dual_1x128<true>(x, rows, cols, q, s, qt, st, stream);
}
extern "C" puro_status puro_quant_w_128x128_group_pow2(const puro_w_item* items, int count,
                                                       void* stream) {
  return quant_w_128x128_group<true>(items, count, stream);
}

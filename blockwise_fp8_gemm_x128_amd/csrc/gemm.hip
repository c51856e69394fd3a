// Blockwise-scaled FP8 GEMMs for gfx950 (CDNA4) on the 16x16x128 FP8 matrix-core instruction.
//
// Method: Paper walkthrough: Puro-2B (ta-paperlens.web.app), section "Lever 2: use blockwise
// FP8 from step zero" — only the linear-layer GEMMs run in FP8, on operands scaled per 1x128
// group along the reduction dimension (activations, gradients) or per 128x128 block (weights).
// Because every scale is constant over one 128-long reduction chunk, each chunk's dot products
// are exact-product FP8 MFMA sums, which are then promoted into an fp32 accumulator:
//     acc += (s_a * s_b) * P_chunk.
//
// All three GEMMs are one kernel template computing
//     C[i][j] = sum_c sA[c][i] * sB(c, j) * sum_{l in chunk c} A[i][l] * B(j, l)
// with A = [I][L] row-major (reduction contiguous) and
//   forward : A = Xq[M][K],   B(j,l) = Wq[j][l]   (row-major [J][L]), sB = sw[j/128][c]
//   dgrad   : A = dYq[M][N],  B(j,l) = Wq[l][j]   ([L][J], read transposed from LDS),
//                                                  sB = sw[c][j/128]
//   wgrad   : A = dYtq[N][M], B(j,l) = Xtq[j][l]  (row-major [J][L]), sB = sxt[c][j]
//
// Work decomposition: a 256-thread block (4 waves, 2x2) owns a 128x128 tile of C; each wave
// owns 64x64 = 4x4 MFMA tiles of 16x16. Per reduction chunk the block stages a 128x128-byte
// tile of A and of B in LDS (double buffered: the next chunk's global loads are in flight while
// the current chunk is multiplied), with the 16-byte pieces of each row XOR-swizzled so that
// fragment reads are spread over the LDS banks.
#include "common.hpp"

namespace puro {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

enum ScaleB : int {
  kScaleBlockRow = 0,  // sB[(j/128) * (L/128) + c]   forward: sw[n/128][kb]
  kScaleBlockCol = 1,  // sB[c * (J/128) + j/128]     dgrad:   sw[nb][k/128]
  kScalePerCol = 2     // sB[c * J + j]               wgrad:   sxt[mb][k]
};

constexpr int kTile = 128;                // C tile edge and reduction chunk
constexpr int kTileBytes = kTile * kTile; // one staged FP8 operand tile

// Row r of a staged tile keeps its eight 16-byte pieces in XOR-permuted order.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ ((row >> 5) << 2)) & 7; }
__device__ __forceinline__ int lds_off(int row, int piece) {
  return row * kTile + ((piece ^ swz(row)) << 4);
}

// Global -> registers: a 128-row x 128-byte tile, 4 pieces of 16 B per thread, 8 lanes per row.
__device__ __forceinline__ void load_tile(v4i (&r)[4], const uint8_t* __restrict__ base,
                                          int64_t ld, int t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = t + 256 * i;
    r[i] = *reinterpret_cast<const v4i*>(base + int64_t(p >> 3) * ld + ((p & 7) << 4));
  }
}

// Registers -> LDS (swizzled).
__device__ __forceinline__ void store_tile(uint8_t* lds, const v4i (&r)[4], int t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = t + 256 * i;
    *reinterpret_cast<v4i*>(lds + lds_off(p >> 3, p & 7)) = r[i];
  }
}

// MFMA operand fragment for 16 rows starting at `row0` of a row-major staged tile: lane l takes
// row row0 + l%16 and reduction bytes [32*(l/16), 32*(l/16)+32).
__device__ __forceinline__ v8i frag_rows(const uint8_t* lds, int row0, int lane) {
  const int row = row0 + (lane & 15);
  const int piece = (lane >> 4) * 2;
  const v4i lo = *reinterpret_cast<const v4i*>(lds + lds_off(row, piece));
  const v4i hi = *reinterpret_cast<const v4i*>(lds + lds_off(row, piece + 1));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Same fragment when the staged tile is stored reduction-major (row = reduction index,
// 128 bytes = output columns): lane l must gather column col0 + l%16 over reduction rows
// [32*(l/16), +32). ds_read_b64_tr_b8 does the gather: in each 16-lane group G, lane
// 16G + 8h + b receives, as byte j, byte b of the 8 bytes addressed by lane 16G + 2j + h.
// So lane 16G + r addresses row 32G + 8i + r/2, bytes [col0 + 8*(r%2), +8), for i = 0..3.
__device__ __forceinline__ v8i frag_cols_tr(const uint8_t* lds, int col0, int lane) {
  const int G = lane >> 4, r = lane & 15;
  const int piece = col0 >> 4;
  v8i f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * G + 8 * i + (r >> 1);
    const uint8_t* p = lds + lds_off(row, piece) + 8 * (r & 1);
    const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p));
    f[2 * i] = v[0];
    f[2 * i + 1] = v[1];
  }
  return f;
}

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

template <bool kBTrans, int kScaleB, bool kOutF32>
__global__ __launch_bounds__(256) void gemm_blockscaled_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, void* __restrict__ Cout, int64_t I, int64_t J, int64_t L,
    int accumulate) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileBytes];

  const int64_t tiles_j = J / kTile;
  const int64_t ti = blockIdx.x / tiles_j;
  const int64_t tj = blockIdx.x % tiles_j;
  const int64_t i0 = ti * kTile, j0 = tj * kTile;
  const int t = threadIdx.x;
  const int w = t >> 6, lane = t & 63;
  const int G = lane >> 4, c16 = lane & 15;
  const int wm = w >> 1, wn = w & 1;
  const int64_t nk = L / kTile;

  v4f acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // Operand tile origins for chunk c.
  const uint8_t* a_base = A + i0 * L;
  auto b_tile = [&](int64_t c) -> const uint8_t* {
    return kBTrans ? B + c * kTile * J + j0 : B + j0 * L + c * kTile;
  };
  const int64_t ldb = kBTrans ? J : L;

  // Scales for chunk c: this lane's rows 4G..4G+3 of each 16-row block, and the B scale(s).
  const int64_t row_base = i0 + wm * 64 + 4 * G;
  const int64_t col_base = j0 + wn * 64 + c16;
  auto load_sa = [&](int64_t c, v4f (&sa)[4]) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      sa[mi] = *reinterpret_cast<const v4f*>(sA + c * I + row_base + 16 * mi);
  };
  auto load_sb = [&](int64_t c, float (&sb)[4]) {
    if (kScaleB == kScalePerCol) {
#pragma unroll
      for (int nj = 0; nj < 4; ++nj) sb[nj] = sB[c * J + col_base + 16 * nj];
    } else {
      const float v = kScaleB == kScaleBlockRow ? sB[tj * nk + c] : sB[c * tiles_j + tj];
#pragma unroll
      for (int nj = 0; nj < 4; ++nj) sb[nj] = v;
    }
  };

  v4f sa_next[4];
  float sb_next[4];
  if (nk > 0) {
    v4i ra[4], rb[4];
    load_tile(ra, a_base, L, t);
    load_tile(rb, b_tile(0), ldb, t);
    load_sa(0, sa_next);
    load_sb(0, sb_next);
    store_tile(lds[0][0], ra, t);
    store_tile(lds[0][1], rb, t);
  }
  __syncthreads();

#pragma clang loop unroll(disable)
  for (int64_t c = 0; c < nk; ++c) {
    const int cur = static_cast<int>(c & 1);
    const bool more = c + 1 < nk;
    v4i ra[4], rb[4];
    if (more) {
      load_tile(ra, a_base + (c + 1) * kTile, L, t);
      load_tile(rb, b_tile(c + 1), ldb, t);
    }
    v4f sa[4];
    float sb[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) sa[mi] = sa_next[mi];
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) sb[nj] = sb_next[nj];
    if (more) {
      load_sa(c + 1, sa_next);
      load_sb(c + 1, sb_next);
    }

    v8i af[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) af[mi] = frag_rows(lds[cur][0], wm * 64 + 16 * mi, lane);
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) {
      const v8i bf = kBTrans ? frag_cols_tr(lds[cur][1], wn * 64 + 16 * nj, lane)
                             : frag_rows(lds[cur][1], wn * 64 + 16 * nj, lane);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const v4f p = mfma_fp8(af[mi], bf);
        const v4f s = sa[mi] * sb[nj];
        acc[mi][nj] += s * p;
      }
    }

    if (more) {
      store_tile(lds[cur ^ 1][0], ra, t);
      store_tile(lds[cur ^ 1][1], rb, t);
    }
    __syncthreads();
  }

  // Epilogue: lane holds rows 4G+v, column c16 of every 16x16 tile.
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = row_base + 16 * mi + v;
        const int64_t col = j0 + wn * 64 + 16 * nj + c16;
        if (kOutF32) {
          float* out = static_cast<float*>(Cout) + row * J + col;
          *out = accumulate ? *out + acc[mi][nj][v] : acc[mi][nj][v];
        } else {
          uint16_t* out = static_cast<uint16_t*>(Cout) + row * J + col;
          *out = static_cast<uint16_t>(f32_to_bf16_rne(acc[mi][nj][v]));
        }
      }
    }
  }
}

template <bool kBTrans, int kScaleB, bool kOutF32>
puro_status launch_gemm(const void* A, const float* sA, const void* B, const float* sB,
                        void* C, int64_t I, int64_t J, int64_t L, int accumulate,
                        void* stream) {
  const int64_t blocks = (I / kTile) * (J / kTile);
  if (blocks > INT32_MAX) return PURO_ERR_SHAPE;
  hipLaunchKernelGGL((gemm_blockscaled_kernel<kBTrans, kScaleB, kOutF32>),
                     dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(A), sA,
                     static_cast<const uint8_t*>(B), sB, C, I, J, L, accumulate);
  return launch_status();
}

}  // namespace
}  // namespace puro

using namespace puro;

extern "C" puro_status puro_fp8_gemm_fwd(const void* xq, const float* sx, const void* wq,
                                         const float* sw, void* y, int64_t M, int64_t N,
                                         int64_t K, void* stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K)) return PURO_ERR_SHAPE;
  const bool out_empty = M == 0 || N == 0;
  const bool red_empty = out_empty || K == 0;
  PURO_TRY(check_ptr(xq, red_empty));
  PURO_TRY(check_ptr(sx, red_empty));
  PURO_TRY(check_ptr(wq, red_empty));
  PURO_TRY(check_ptr(sw, red_empty));
  PURO_TRY(check_ptr(y, out_empty));
  if (out_empty) return PURO_OK;
  return launch_gemm<false, kScaleBlockRow, false>(xq, sx, wq, sw, y, M, N, K, 0, stream);
}

extern "C" puro_status puro_fp8_gemm_dgrad(const void* dyq, const float* sdy, const void* wq,
                                           const float* sw, void* dx, int64_t M, int64_t N,
                                           int64_t K, void* stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K)) return PURO_ERR_SHAPE;
  const bool out_empty = M == 0 || K == 0;
  const bool red_empty = out_empty || N == 0;
  PURO_TRY(check_ptr(dyq, red_empty));
  PURO_TRY(check_ptr(sdy, red_empty));
  PURO_TRY(check_ptr(wq, red_empty));
  PURO_TRY(check_ptr(sw, red_empty));
  PURO_TRY(check_ptr(dx, out_empty));
  if (out_empty) return PURO_OK;
  return launch_gemm<true, kScaleBlockCol, false>(dyq, sdy, wq, sw, dx, M, K, N, 0, stream);
}

extern "C" puro_status puro_fp8_gemm_wgrad(const void* dytq, const float* sdyt, const void* xtq,
                                           const float* sxt, float* dw, int64_t M, int64_t N,
                                           int64_t K, int accumulate, void* stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K)) return PURO_ERR_SHAPE;
  if (accumulate != 0 && accumulate != 1) return PURO_ERR_ARG;
  const bool out_empty = N == 0 || K == 0;
  const bool red_empty = out_empty || M == 0;
  PURO_TRY(check_ptr(dytq, red_empty));
  PURO_TRY(check_ptr(sdyt, red_empty));
  PURO_TRY(check_ptr(xtq, red_empty));
  PURO_TRY(check_ptr(sxt, red_empty));
  PURO_TRY(check_ptr(dw, out_empty));
  if (out_empty) return PURO_OK;
  return launch_gemm<false, kScalePerCol, true>(dytq, sdyt, xtq, sxt, dw, N, K, M, accumulate,
                                                stream);
}

// Blockwise-scaled FP8 GEMMs for gfx950 (CDNA4) on the 16x16x128 FP8 matrix-core instruction.
//
// Method: Paper walkthrough: Puro-2B (ta-paperlens.web.app), section "Lever 2: use blockwise
// FP8 from step zero" — only the linear-layer GEMMs run in FP8, on operands scaled per 1x128
// group along the reduction dimension (activations, gradients) or per 128x128 block (weights).
// Every scale is constant over one 128-long reduction chunk, so each chunk's dot products are
// taken on the matrix cores (exact FP8 products, fp32 sums) and then promoted into an fp32
// accumulator:   acc += (s_a * s_b) * P_chunk.
//
// All three GEMMs are one kernel template computing
//     C[i][j] = sum_c sA[c][i] * sB(c, j) * sum_{l in chunk c} A[i][l] * B(j, l)
// with A = [I][L] row-major (reduction contiguous) and
//   forward : A = Xq[M][K],   B(j,l) = Wq[j][l]  (row-major [J][L]),  sB = sw[j/128][c]
//   dgrad   : A = dYq[M][N],  B(j,l) = Wq[l][j]  ([L][J], gathered transposed from LDS),
//                                                 sB = sw[c][j/128]
//   wgrad   : A = dYtq[N][M], B(j,l) = Xtq[j][l] (row-major [J][L]),  sB = sxt[c][j]
//
// Decomposition. A block owns a BM x BN tile of C and WAVES_M x WAVES_N waves; each wave owns
// a WM x WN sub-tile = (WM/16) x (WN/16) MFMA tiles of 16x16. The reduction runs in 128-wide
// chunks through a two-stage LDS pipeline: while chunk c is multiplied out of one stage, chunk
// c+1 (A tile, B tile and the A/B scale rows) streams into the other stage with
// global_load_lds_dwordx4, which writes LDS directly (no VGPR staging, no ds_write). One barrier
// per chunk separates "stage landed" from "stage free". Each 128-byte row of a staged operand
// keeps its 16-byte pieces XOR-permuted so fragment reads spread over the LDS banks.
//
// Block order: workgroups are dispatched round-robin over the 8 XCDs, so the block id is first
// remapped so that consecutive tiles run on one XCD (sharing that XCD's L2), and tiles are
// walked in bands of 8 tile-rows, column by column, so concurrently running tiles share A and B
// panels.
#include "common.hpp"

namespace puro {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) void lds_void;

enum Mode : int { kFwd = 0, kDgrad = 1, kWgrad = 2 };

constexpr int kChunk = 128;       // reduction chunk = quantisation group
constexpr int kSlab = 128 * 128;  // bytes of one 128-row x 128-byte staged slab
constexpr int kGroupRows = 8;     // tile-rows per band of the block order

template <int kMode, int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct Cfg {
  static constexpr int mode = kMode;
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int MI = WM / 16, NJ = WN / 16;
  static constexpr bool kBTrans = kMode == kDgrad;
  static constexpr bool kPerColScale = kMode == kWgrad;
  static constexpr bool kOutF32 = kMode == kWgrad;
  // stage layout in bytes: A rows | B rows (or B slabs) | A scales | B scales (per-column only)
  static constexpr int kAOff = 0;
  static constexpr int kBOff = BM * kChunk;
  static constexpr int kSAOff = kBOff + BN * kChunk;
  static constexpr int kSBOff = kSAOff + BM * 4;
  static constexpr int kStageBytes = kSBOff + (kPerColScale ? BN * 4 : 0);
  static_assert(BM % 128 == 0 && BN % 128 == 0, "tiles are whole 128x128 blocks");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns lie in one 128-column block");
  static_assert(WM <= 128 && 128 % WM == 0, "a wave's rows lie in one 128-row half");
  static_assert((BM / 8) % kWaves == 0 && (BN / 8) % kWaves == 0, "even DMA split");
  static_assert(BM / 4 <= 64 && BN / 4 <= 64, "one DMA instruction per scale row");
  static_assert(WM % 64 == 0 || WM == 16 * MI, "row-block swizzle parity is per-block");
  static_assert(!kBTrans || WN == 64, "reduction-major B fragment offsets assume WN = 64");
};

// Row r of a staged 128-byte-row array keeps its eight 16-byte pieces in XOR-permuted order.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ ((row >> 5) << 2)) & 7; }

__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// 16 bytes per lane from global memory straight into LDS through a buffer resource: lane i's
// bytes (at base + voff_i + soff) land at lds_dst + 16 * i (lds_dst is wave-uniform). Offsets
// at or beyond the resource's byte count read as zero, which covers the invalid half of edge
// tiles without any clamping.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw, untyped 32-bit-offset buffer (gfx9 family)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes > int64_t(0xffffffff) ? 0xffffffffu : static_cast<uint32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n),
                                           kRsrcWord3);
}

__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, static_cast<int>(voff),
                                           static_cast<int>(soff), 0, 0);
}

template <class C>
struct Loader {
  static constexpr int kAInstr = C::BM / 8 / C::kWaves;  // DMA instructions per wave, A tile
  static constexpr int kBInstr = C::BN / 8 / C::kWaves;  // and B tile

  // Instruction k of wave w copies staged rows [8q, 8q+8), q = w + kWaves*k; lane l takes row
  // 8q + l/8 and physical piece l%8, i.e. logical piece (l%8) ^ swz(row). That XOR term does not
  // depend on k, so all of a lane's instructions share one per-lane offset; the row offset of
  // instruction k and the chunk offset are wave-uniform (scalar offset / resource base).
  const uint8_t* A;
  const uint8_t* B;
  const float* sA;
  const float* sB;
  int64_t I, J, L, i0, j0;
  rsrc_t ra, rb;          // per-tile resources (A, and row-major B)
  uint32_t a_voff, b_voff;
  int wave, lane;
  const float* sb_block;  // block modes: the wave's block scale of chunk 0 (uniform)
  int64_t sb_block_step;

  __device__ __forceinline__ void init(int wn) {
    const int r8 = lane >> 3, p8 = lane & 7;
    const int xr = ((8 * wave + r8) >> 1 ^ ((8 * wave + r8) >> 5) << 2) & 7;  // swz, any k
    ra = make_rsrc(A + i0 * L, (I - i0) * L);
    a_voff = static_cast<uint32_t>(r8 * L + ((p8 ^ xr) << 4));
    if (C::kBTrans) {
      b_voff = static_cast<uint32_t>(r8 * J + ((p8 ^ xr) << 4));
    } else {
      rb = make_rsrc(B + j0 * L, (J - j0) * L);
      b_voff = static_cast<uint32_t>(r8 * L + ((p8 ^ xr) << 4));
    }
    const int64_t jb = imin64(j0 + (wave % C::WAVES_N) * C::WN, J - 1) / 128;
    (void)wn;
    if (C::mode == kFwd) {
      sb_block = sB + jb * (L / kChunk);
      sb_block_step = 1;
    } else {
      sb_block = sB + jb;
      sb_block_step = J / 128;
    }
  }

  // Enqueue chunk c into `stage` (every wave issues its share; DMA writes LDS directly).
  __device__ __forceinline__ void issue(uint8_t* stage, int64_t c) const {
#pragma unroll
    for (int k = 0; k < kAInstr; ++k) {
      const int q = wave + C::kWaves * k;
      dma16(ra, a_voff, static_cast<uint32_t>(8 * q * L + c * kChunk),
            stage + C::kAOff + 8 * q * kChunk);
    }
    if (C::kBTrans) {
      // staged B = BN/128 slabs of 128 reduction rows x 128 columns; slab s holds columns
      // j0 + 128 s .. +127 and its row rr is reduction row rr of the chunk
      const uint8_t* base = B + c * kChunk * J + j0;
      const rsrc_t rbc = make_rsrc(base, (L - c * kChunk) * J - j0);
#pragma unroll
      for (int k = 0; k < kBInstr; ++k) {
        const int q = wave + C::kWaves * k;
        const int sl = q >> 4, qq = q & 15;
        dma16(rbc, b_voff, static_cast<uint32_t>(8 * qq * J + 128 * sl),
              stage + C::kBOff + 8 * q * kChunk);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kBInstr; ++k) {
        const int q = wave + C::kWaves * k;
        dma16(rb, b_voff, static_cast<uint32_t>(8 * q * L + c * kChunk),
              stage + C::kBOff + 8 * q * kChunk);
      }
    }
    if (wave == 0 && lane < C::BM / 4)
      dma16(make_rsrc(sA + c * I + i0, (I - i0) * 4), 16 * lane, 0, stage + C::kSAOff);
    if (C::kPerColScale && wave == (1 % C::kWaves) && lane < C::BN / 4)
      dma16(make_rsrc(sB + c * J + j0, (J - j0) * 4), 16 * lane, 0, stage + C::kSBOff);
  }
};

// Per-lane LDS byte offsets of this wave's fragment reads, fixed for the whole kernel.
// For 16 consecutive staged rows R0 + r (R0 a multiple of 16) the swizzle is
// swz(R0 + r) = ((r >> 1) & 7) ^ 4 * ((R0 >> 5) & 1): a per-lane term and a term known per row
// block, so two variants (f = 0 / 4) cover every row block of the wave.
template <class C>
struct FragOffsets {
  int a[2][2];      // [f/4][half]: A rows, wave-relative
  int b[2][2];      // same for row-major B
  int bt[2][4];     // reduction-major B: [i & 1][nj]
  int sa;           // this lane's 4 A scales (wave-relative)
  int sb;           // this lane's B scale column base (per-column mode)

  __device__ __forceinline__ void init(int wm, int wn, int lane) {
    const int G = lane >> 4, r = lane & 15;
    for (int f = 0; f < 2; ++f)
      for (int e = 0; e < 2; ++e) {
        const int x = ((2 * G + e) ^ ((r >> 1) & 7) ^ (4 * f)) << 4;
        a[f][e] = C::kAOff + (wm * C::WM + r) * kChunk + x;
        b[f][e] = C::kBOff + (wn * C::WN + r) * kChunk + x;
      }
    // Reduction-major B (dgrad): fragment (nj, i) reads slab (col >> 7), row 32G + 8i + r/2,
    // piece (col & 127) >> 4 = 4 * (wn & 1) + nj when WN = 64, swizzled by
    // swz(row) = (4i & 7) ^ (r >> 2) ^ 4 * (G & 1).
    const int y = (r >> 2) ^ (4 * ((G & 1) ^ ((wn * C::WN >> 6) & 1)));
    const int slab = ((wn * C::WN) >> 7) * kSlab;
    for (int io = 0; io < 2; ++io)
      for (int nj = 0; nj < 4; ++nj)
        bt[io][nj] = C::kBOff + slab + (32 * G + (r >> 1)) * kChunk + 8 * (r & 1) +
                     ((nj ^ y ^ (4 * io)) << 4);
    sa = C::kSAOff + (wm * C::WM + 4 * G) * 4;
    sb = C::kSBOff + (wn * C::WN + r) * 4;
  }
};

template <int kOff>
__device__ __forceinline__ v4i lds_v4i(const uint8_t* stage, int off) {
  return *reinterpret_cast<const v4i*>(stage + off + kOff);
}

// A-type fragment: 16 rows starting at wave row 16*mi.
template <class C, int mi>
__device__ __forceinline__ v8i frag_a(const uint8_t* stage, const FragOffsets<C>& o) {
  constexpr int f = (mi >> 1) & 1;  // (16 mi >> 5) & 1; the wave's row origin is a multiple of 64
  const v4i lo = lds_v4i<16 * mi * kChunk>(stage, o.a[f][0]);
  const v4i hi = lds_v4i<16 * mi * kChunk>(stage, o.a[f][1]);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <class C, int nj>
__device__ __forceinline__ v8i frag_b(const uint8_t* stage, const FragOffsets<C>& o) {
  if (C::kBTrans) {
    v8i f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_v2i*)(stage + o.bt[i & 1][nj] + 8 * i * kChunk));
      f[2 * i] = v[0];
      f[2 * i + 1] = v[1];
    }
    return f;
  } else {
    constexpr int f = (nj >> 1) & 1;
    const v4i lo = lds_v4i<16 * nj * kChunk>(stage, o.b[f][0]);
    const v4i hi = lds_v4i<16 * nj * kChunk>(stage, o.b[f][1]);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

template <class C, int mi>
__device__ __forceinline__ v4f scale_a(const uint8_t* stage, const FragOffsets<C>& o) {
  return *reinterpret_cast<const v4f*>(stage + o.sa + 16 * mi * 4);
}

// Software pipeline over the MI x NJ MFMA tiles of a chunk, flattened as k = mi * NJ + nj:
// step k issues MFMA k and then promotes MFMA k - NJ (same column, previous row block), whose
// result is ready by then, so the promotion FMAs run on the vector ALU while the matrix core
// works through the next products. Only NJ + 1 product vectors are live at once. The next row
// block's A fragment and scales are fetched from LDS at the start of each row block.
template <class C>
struct ChunkState {
  static constexpr int kWin = C::NJ + 1;
  v8i bf[C::NJ];
  float sbv[C::NJ];
  v4f p[kWin];
  v8i af_cur, af_next;
  v4f sa_cur, sa_next, sa_prev;
};

template <class C, int k>
__device__ __forceinline__ void chunk_step(const uint8_t* stage, const FragOffsets<C>& o,
                                           ChunkState<C>& st, float sb_blk,
                                           v4f (&acc)[C::MI][C::NJ]) {
  constexpr int kTiles = C::MI * C::NJ;
  if constexpr (k < kTiles + C::NJ) {
    constexpr int mi = k / C::NJ, nj = k % C::NJ;
    constexpr int kWin = ChunkState<C>::kWin;
    if constexpr (k < kTiles) {
      if constexpr (nj == 0 && mi + 1 < C::MI) {
        st.af_next = frag_a<C, mi + 1>(stage, o);
        st.sa_next = scale_a<C, mi + 1>(stage, o);
      }
      st.p[k % kWin] = mfma_fp8(st.af_cur, st.bf[nj]);
    }
    if constexpr (k >= C::NJ) {
      constexpr int kp = k - C::NJ;
      constexpr int mp = kp / C::NJ, np = kp % C::NJ;
      const v4f s = C::kPerColScale ? st.sa_prev * st.sbv[np] : st.sa_prev * sb_blk;
      acc[mp][np] += s * st.p[kp % kWin];
      // Pin the promoted accumulator here: without this, IR-level sinking defers whole chunks of
      // promotions past the next barrier and keeps their products live (register spills).
      asm volatile("" : "+v"(acc[mp][np]));
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (nj == C::NJ - 1) {  // row block mi done: rotate the A fragment and scales
      st.sa_prev = st.sa_cur;
      if constexpr (mi + 1 < C::MI) {
        st.af_cur = st.af_next;
        st.sa_cur = st.sa_next;
      }
    }
    chunk_step<C, k + 1>(stage, o, st, sb_blk, acc);
  }
}

template <class C, int nj>
__device__ __forceinline__ void load_bf(const uint8_t* stage, const FragOffsets<C>& o,
                                        ChunkState<C>& st, float sb_blk) {
  if constexpr (nj < C::NJ) {
    st.bf[nj] = frag_b<C, nj>(stage, o);
    st.sbv[nj] =
        C::kPerColScale ? *reinterpret_cast<const float*>(stage + o.sb + 64 * nj) : sb_blk;
    load_bf<C, nj + 1>(stage, o, st, sb_blk);
  }
}

// One 128-wide reduction chunk out of a landed stage.
template <class C>
__device__ __forceinline__ void compute_chunk(const uint8_t* stage, float sb_blk,
                                              const FragOffsets<C>& o,
                                              v4f (&acc)[C::MI][C::NJ]) {
  ChunkState<C> st;
  load_bf<C, 0>(stage, o, st, sb_blk);
  st.af_cur = frag_a<C, 0>(stage, o);
  st.sa_cur = scale_a<C, 0>(stage, o);
  chunk_step<C, 0>(stage, o, st, sb_blk, acc);
}

template <class C>
__device__ __forceinline__ void gemm_body(const uint8_t* __restrict__ A,
                                          const float* __restrict__ sA,
                                          const uint8_t* __restrict__ B,
                                          const float* __restrict__ sB, void* __restrict__ Cout,
                                          int64_t I, int64_t J, int64_t L, int accumulate,
                                          uint8_t* stage0, uint8_t* stage1) {
  const int64_t tiles_i = (I + C::BM - 1) / C::BM;
  const int64_t tiles_j = (J + C::BN - 1) / C::BN;
  const int64_t nwg = tiles_i * tiles_j;
  int64_t b = blockIdx.x;
  if ((nwg & 7) == 0) b = (b & 7) * (nwg >> 3) + (b >> 3);
  const int64_t band = b / (kGroupRows * tiles_j);
  const int64_t band_rows = imin64(kGroupRows, tiles_i - band * kGroupRows);
  const int64_t local = b - band * kGroupRows * tiles_j;
  const int64_t ti = band * kGroupRows + local % band_rows;
  const int64_t tj = local / band_rows;
  const int64_t i0 = ti * C::BM, j0 = tj * C::BN;

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int64_t nk = L / kChunk;

  Loader<C> ld;
  ld.A = A;
  ld.B = B;
  ld.sA = sA;
  ld.sB = sB;
  ld.I = I;
  ld.J = J;
  ld.L = L;
  ld.i0 = i0;
  ld.j0 = j0;
  ld.wave = wave;
  ld.lane = lane;
  ld.init(wn);
  FragOffsets<C> fo;
  fo.init(wm, wn, lane);

  v4f acc[C::MI][C::NJ];
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj) acc[mi][nj] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if (nk > 0) ld.issue(stage0, 0);
  float sb_next = (!C::kPerColScale && nk > 0) ? ld.sb_block[0] : 0.0f;

  // Chunks go in pairs (stage0 then stage1) so that each stage is a distinct LDS object; an odd
  // last chunk is handled after the loop. Every half: wait for this wave's DMA, barrier (the
  // stage has landed for all waves, and the other stage is no longer being read), enqueue the
  // next chunk into the other stage, multiply out of this one.
  auto half = [&](uint8_t* cur, uint8_t* nxt, int64_t c) {
    const float sb = sb_next;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (c + 1 < nk) {
      ld.issue(nxt, c + 1);
      if (!C::kPerColScale) sb_next = ld.sb_block[(c + 1) * ld.sb_block_step];
    }
    compute_chunk<C>(cur, sb, fo, acc);
  };
  int64_t c = 0;
  for (; c + 1 < nk; c += 2) {
    half(stage0, stage1, c);
    half(stage1, stage0, c + 1);
  }
  if (c < nk) half(stage0, stage1, c);

  // Epilogue: lane holds rows 4G+v and column c16 of every 16x16 tile.
  const int G = lane >> 4, c16 = lane & 15;
  const int64_t r0 = i0 + wm * C::WM, q0 = j0 + wn * C::WN;
  if (r0 >= I || q0 >= J) return;  // this wave lies in the invalid half of an edge tile
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) {
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = r0 + 16 * mi + 4 * G + v;
        const int64_t col = q0 + 16 * nj + c16;
        if (C::kOutF32) {
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

using FwdBig = Cfg<kFwd, 256, 256, 2, 4>;
using DgradBig = Cfg<kDgrad, 256, 256, 2, 4>;
using WgradBig = Cfg<kWgrad, 256, 256, 2, 4>;

#define PURO_GEMM_KERNEL(NAME, CFG)                                                        \
  __global__ __launch_bounds__(CFG::kThreads) void NAME(                                   \
      const uint8_t* __restrict__ A, const float* __restrict__ sA,                         \
      const uint8_t* __restrict__ B, const float* __restrict__ sB, void* __restrict__ Cout, \
      int64_t I, int64_t J, int64_t L, int accumulate) {                                   \
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[CFG::kStageBytes];            \
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[CFG::kStageBytes];            \
    gemm_body<CFG>(A, sA, B, sB, Cout, I, J, L, accumulate, stage0, stage1);               \
  }

PURO_GEMM_KERNEL(gemm_fwd_256x256, FwdBig)
PURO_GEMM_KERNEL(gemm_dgrad_256x256, DgradBig)
PURO_GEMM_KERNEL(gemm_wgrad_256x256, WgradBig)

typedef void (*GemmKernel)(const uint8_t*, const float*, const uint8_t*, const float*, void*,
                           int64_t, int64_t, int64_t, int);

template <class C>
puro_status launch(GemmKernel k, const void* A, const float* sA, const void* B, const float* sB,
                   void* Cout, int64_t I, int64_t J, int64_t L, int accumulate, void* stream) {
  const int64_t blocks = ((I + C::BM - 1) / C::BM) * ((J + C::BN - 1) / C::BN);
  if (blocks > INT32_MAX) return PURO_ERR_SHAPE;
  hipLaunchKernelGGL(k, dim3(static_cast<uint32_t>(blocks)), dim3(C::kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(A), sA,
                     static_cast<const uint8_t*>(B), sB, Cout, I, J, L, accumulate);
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
  return launch<FwdBig>(gemm_fwd_256x256, xq, sx, wq, sw, y, M, N, K, 0, stream);
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
  return launch<DgradBig>(gemm_dgrad_256x256, dyq, sdy, wq, sw, dx, M, K, N, 0, stream);
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
  return launch<WgradBig>(gemm_wgrad_256x256, dytq, sdyt, xtq, sxt, dw, N, K, M, accumulate,
                          stream);
}

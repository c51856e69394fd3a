// Blockwise-scaled FP8 GEMMs for gfx950 (CDNA4) on the 16x16x128 FP8 matrix-core instruction.
//
// Method: Paper walkthrough: Puro-2B (ta-paperlens.web.app), section "Lever 2: use blockwise
// FP8 from step zero" — only the linear-layer GEMMs run in FP8, on operands scaled per 1x128
// group along the reduction dimension (activations, gradients) or per 128x128 block (weights).
// Every scale is constant over one 128-long reduction chunk, so each chunk's dot products are
// taken on the matrix cores (exact FP8 products, fp32 sums) and then promoted into an fp32
// accumulator:   acc += (s_a * s_b) * P_chunk.
// The power-of-two variant (a library option: scales 2^e) hands each operand row's exponent
// to the scaled FP8 instruction instead, which applies it and accumulates every chunk itself.
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
// buffer_load_dwordx4 ... lds, which writes LDS directly (no VGPR staging, no ds_write). One
// barrier per chunk separates "stage landed" from "stage free". In the 8-wave tiles only half of
// the waves issue a given chunk's DMA, the halves alternating by chunk parity: the issue is
// held up by the CU's memory pipeline (a 256x256 chunk is 64 KB), and the two waves sharing a
// SIMD are in different halves, so one of them keeps the matrix core busy meanwhile. The
// issuing half sends its A rows right after the barrier and its B rows after the chunk's first
// row block of products.
//
// Each 128-byte row of a staged operand keeps its eight 16-byte pieces XOR-permuted (piece p at
// slot p ^ swz(row)). The two swizzles below were chosen by measurement on MI355X
// (SQ_LDS_BANK_CONFLICT of each candidate's exact read pattern): both the 16-byte fragment reads
// (16 rows x 4 lane groups) and the 8-byte transposed reads (4 lane groups x 8 rows x 2 halves)
// run with no bank-conflict cycles, where the unswizzled layout costs 12 and 14 cycles per read
// instruction.
//
// Epilogue: the fragment layout leaves four adjacent results per lane, so stores written
// straight from the accumulators cover a quarter (bf16) or half (fp32) cache line per row.
// Waves 64 columns wide therefore restage their block through LDS (the stage the last chunk did
// not use) and store whole rows, 16 bytes per lane.
//
// Block order: workgroups are dispatched round-robin over the 8 XCDs, so the block id is first
// remapped so that consecutive tiles run on one XCD (sharing that XCD's L2), and tiles are
// walked in bands of 8 tile-rows, column by column, so concurrently running tiles share A and B
// panels.
//
// Split reduction: a weight gradient whose 128x128 tiles would leave the four-wave blocks one
// wave per SIMD (at most one tile per CU) runs two groups of four waves per tile instead, group
// g multiplying out chunks g, g+2, g+4, ... from stages of its own; group 1 then hands its
// partial sums to group 0 through LDS, which adds them in a fixed order and stores the tile.
#include <type_traits>

#include "common.hpp"
#include "debug.hpp"
#include "dma_offsets.hpp"

namespace puro {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
// LDS pointers keep their address space from the kernel entry down, so no generic-to-LDS
// conversions (with their null checks) appear inside the pipeline.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4i lds_v4i_t;
typedef __attribute__((address_space(3))) v4f lds_v4f;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) void lds_void;

enum Mode : int { kFwd = 0, kDgrad = 1, kWgrad = 2 };

constexpr int kChunk = 128;       // reduction chunk = quantisation group
constexpr int kSlab = 128 * 128;  // bytes of one 128-row x 128-byte staged slab
// Tile-rows per band of the block order, for an output `tiles_j` tiles wide: for the forward
// and data-gradient 256x256 tiles 2 up to 24 tile columns and 4 beyond, 8 for the others
// (measured on the linear-stack step, same box, alternated: from 4 to 2 the 16-column qkv
// forward went 62.8 -> 61.1 us and the 24-column down data gradient 91.3 -> 89.7 us, while the
// 48-column gate_up forward went 169.0 -> 169.8 us; the 8-column shapes did not move).
template <int kMode, int BM>
__device__ __forceinline__ int64_t band_rows(int64_t tiles_j) {
  if constexpr (kMode != kWgrad && BM == 256) return tiles_j <= 24 ? 2 : 4;
  return 8;
}

template <int kMode, int BM_, int BN_, int WAVES_M_, int WAVES_N_, bool kPow2_ = false>
struct Cfg {
  static constexpr int mode = kMode;
  static constexpr bool kPow2 = kPow2_;  // power-of-two scales, applied by the matrix cores
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
  static constexpr int kScaleArea = 1024;  // one 64-lane x 16-byte DMA; rows beyond BM read 0
  static constexpr int kSBOff = kSAOff + kScaleArea;
  static constexpr int kStageBytes = kSBOff + (kPerColScale ? kScaleArea : 0);
  static_assert((BM % 128 == 0 && BN % 128 == 0) || kPerColScale,
                "block-scaled tiles are whole 128x128 blocks");
  static_assert(WN % 16 == 0 && (kPerColScale || (WN <= 128 && 128 % WN == 0)),
                "a wave's columns lie in one 128-column scale block");
  static_assert(WM <= 128 && WM % 16 == 0, "a wave's rows are whole 16-row fragments");
  static_assert((BM / 8) % kWaves == 0 && (BN / 8) % kWaves == 0, "even DMA split");
  static_assert(BM * 4 <= kScaleArea && BN * 4 <= kScaleArea, "one DMA per scale row");
  static_assert(!kBTrans || WN == 64, "reduction-major B fragment offsets assume WN = 64");
};

// Swizzle of row-major staged operands (A, and B of forward / wgrad): row bits 0-1 -> slot bits
// 1-2, row bit 3 -> slot bit 0. It depends on row bits 0-3 only, as the loader and the fragment
// offsets below require.
__device__ __forceinline__ int swz_rows(int row) { return ((row & 3) << 1) | ((row >> 3) & 1); }
// Swizzle of reduction-major slabs (B of dgrad): row bits 1-2 -> slot bits 0-1, row bit 5 ->
// slot bit 2. It ignores row bits 3-4, as the transposed fragment offsets below require.
__device__ __forceinline__ int swz_slab(int row) { return ((row >> 1) & 3) | ((row >> 3) & 4); }

__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

// A 64-bit value that is the same in every lane, moved to scalar registers. The tile origin is
// computed with 64-bit divisions that the compiler expands on the vector ALU; without this it
// can lose track of the result being uniform and wrap every buffer load that uses it in a
// loop over distinct lane values.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// 16 bytes per lane from global memory straight into LDS through a buffer resource: lane i's
// bytes (at base + voff_i + soff) land at lds_dst + 16 * i (lds_dst and soff are wave-uniform).
// Tiles that lie partly outside an operand pass the whole offset per lane (soff = 0), so the
// range check sees the row (and column) each lane addresses: offsets at or beyond the resource's
// byte count read as zero, which covers the invalid part of edge tiles without clamping and
// without reading past a tensor's end. Tiles wholly inside the operand address only its own
// bytes and need no check: in the weight-gradient kernels their loads keep the wave-uniform part
// of the offset in soff, which saves a vector add per load (those kernels are bound by their
// vector ALU).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw, untyped 32-bit-offset buffer (gfx9 family)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes > int64_t(0xffffffff) ? 0xffffffffu : static_cast<uint32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n),
                                           kRsrcWord3);
}

__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, lds_u8* lds_dst,
                                      uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, static_cast<int>(voff),
                                           static_cast<int>(soff), 0, 0);
}

// A chunk's lane offset: the lane part plus the chunk's column offset, hidden from the
// optimiser so that it does not keep one hoisted register per load of the chunk (each load adds
// its wave-uniform row-group offset to this one register instead).
__device__ __forceinline__ uint32_t chunk_lane_offset(uint32_t lane_part, int64_t c) {
  uint32_t v = lane_part + static_cast<uint32_t>(c * 128);
  asm volatile("" : "+v"(v));
  return v;
}

template <class C, bool kScalarRowOffsets_ = C::mode == kWgrad>
struct Loader {
  // 8-wave tiles alternate the DMA between the two halves of the block by chunk parity (waves w
  // and w + 4 share a SIMD, so while one of them is held up feeding the memory pipeline the
  // other keeps the matrix core busy); 4-wave tiles spread every chunk over all their waves.
  static constexpr bool kPingPong = C::kWaves == 8;
  static constexpr int kIssuers = kPingPong ? C::kWaves / 2 : C::kWaves;
  static constexpr int kAInstr = C::BM / 8 / kIssuers;  // DMA instructions per issuing wave, A
  static constexpr int kBInstr = C::BN / 8 / kIssuers;  // and B tile
  // Interior tiles take the scalar-offset form in the one-group weight-gradient kernels only.
  // Measured on MI355X (same box, alternated): the 4-wave 128x128 weight gradient 3.4 % faster,
  // 192x256 1.7 %, 256x192 0.5 %; the split-reduction kernel 3.8 % slower (38 scalar registers
  // spilled to vector lanes instead of 25), the forward and data-gradient kernels 0.5 % and
  // 1.6 % slower (0 -> 19 and 19 -> 34 spilled).
  static constexpr bool kScalarRowOffsets = kScalarRowOffsets_;

  // Instruction k of issuing wave w copies staged rows [8q, 8q+8), q = w + kIssuers*k; lane l
  // takes row 8q + l/8 and physical piece l%8, i.e. logical piece (l%8) ^ swz(row). For
  // row-major operands swz_rows(8q + l/8) depends only on l and on q & 1 = w & 1 (kIssuers is
  // even), so all of a lane's instructions share one lane part of the offset, to which each
  // load adds its wave-uniform row-group and chunk part; for slabs swz_slab depends on k as well
  // and each instruction keeps its own whole offset (the chunk is in the resource base).
  const uint8_t* A;
  const uint8_t* B;
  const float* sA;
  const float* sB;
  int64_t I, J, L, i0, j0;
  rsrc_t ra, rb;          // per-tile resources (A, and row-major B)
  uint32_t a_voff, b_voff;
  bool a_inside, b_inside;  // the tile's rows of A (of row-major B) all lie inside the operand
  uint32_t bt_voff[kBInstr];  // reduction-major B: per instruction
  int wave, lane;
  const float* sb_block;  // block modes: the wave's block scale of chunk 0 (uniform)
  int64_t sb_block_step;
  rsrc_t rsb;             // block modes: resource over the wave's block scales of every chunk

  __device__ __forceinline__ void init(int wn) {
    static_assert(kIssuers % 2 == 0, "row-major DMA swizzle assumes an even issuer count");
    static_assert((C::BM / 8) % kIssuers == 0 && (C::BN / 8) % kIssuers == 0, "even DMA split");
    const int w = kPingPong ? wave % kIssuers : wave;  // this wave's place among the issuers
    const int r8 = lane >> 3, p8 = lane & 7;
    const int xr = swz_rows(8 * w + r8);  // = swz_rows(8q + r8) for every instruction k
    ra = make_rsrc(A + i0 * L, (I - i0) * L);
    a_voff = dma::rows_lane(r8, p8 ^ xr, L);
    a_inside = kScalarRowOffsets && I - i0 >= C::BM;
    b_inside = kScalarRowOffsets && J - j0 >= C::BN;
    if (C::kBTrans) {
#pragma unroll
      for (int k = 0; k < kBInstr; ++k) {
        const int q = w + kIssuers * k;
        const int rr = 8 * (q & 15) + r8;  // row inside its slab
        bt_voff[k] = dma::slab_lane(q, r8, p8 ^ swz_slab(rr), J);
      }
    } else {
      rb = make_rsrc(B + j0 * L, (J - j0) * L);
      b_voff = dma::rows_lane(r8, p8 ^ xr, L);
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
    const int64_t nk = L / kChunk;
    rsb = make_rsrc(sb_block, nk > 0 ? ((nk - 1) * sb_block_step + 1) * 4 : 0);
  }

  // Block scale of chunk c (block modes), read with a vector load: a scalar load would share
  // the counter of the LDS fragment reads and, since scalar loads may return out of order, make
  // every wait on those reads a wait for all of them (measured: each chunk's first products
  // waited for the whole chunk's fragments). The value is used one chunk later, after the
  // barrier's wait for all vector memory.
  __device__ __forceinline__ float block_scale(int64_t c) const {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(
                   rsb, static_cast<int>(c * sb_block_step * 4), 0, 0));
  }

  // Enqueue chunk c into `stage` (the DMA writes LDS directly). A 4-wave block issues all of it
  // here, every wave its share. In an 8-wave block only the issuing half takes part, and here
  // only its A rows and scale rows: its B rows follow from issue_second, after the first row
  // block's products, so that the issuing waves never stall on 16 loads in a row (measured: with
  // one burst, the long-reduction data gradient ran 6 % slower in the model step).
  __device__ __forceinline__ void issue(lds_u8* stage, int64_t c) const {
    if constexpr (kPingPong) {
      if (wave / kIssuers == static_cast<int>(c & 1)) issue_as_a(stage, c, wave % kIssuers);
    } else {
      // The same share written out with the wave index itself: routed through the issuing-wave
      // functions below, the compiler merged the two scale loads of the 4-wave weight-gradient
      // kernel into one with a selected source and that kernel ran 7-9 % slower (MI355X).
      if (a_inside) {
#pragma unroll
        for (int k = 0; k < kAInstr; ++k) {
          const int q = wave + C::kWaves * k;
          dma16(ra, a_voff, stage + C::kAOff + 8 * q * kChunk, dma::rows_group(q, L, c));
        }
      } else {
        const uint32_t av = chunk_lane_offset(a_voff, c);
#pragma unroll
        for (int k = 0; k < kAInstr; ++k) {
          const int q = wave + C::kWaves * k;
          dma16(ra, av + dma::rows_group(q, L, 0), stage + C::kAOff + 8 * q * kChunk);
        }
      }
      if (C::kBTrans) {
        // staged B = BN/128 slabs of 128 reduction rows x 128 columns; slab s holds columns
        // j0 + 128 s .. +127 and its row rr is reduction row rr of the chunk
        const uint8_t* base = B + c * kChunk * J + j0;
        const rsrc_t rbc = make_rsrc(base, (L - c * kChunk) * J - j0);
#pragma unroll
        for (int k = 0; k < kBInstr; ++k) {
          const int q = wave + C::kWaves * k;
          dma16(rbc, bt_voff[k], stage + C::kBOff + 8 * q * kChunk);
        }
      } else if (b_inside) {
#pragma unroll
        for (int k = 0; k < kBInstr; ++k) {
          const int q = wave + C::kWaves * k;
          dma16(rb, b_voff, stage + C::kBOff + 8 * q * kChunk, dma::rows_group(q, L, c));
        }
      } else {
        const uint32_t bv = chunk_lane_offset(b_voff, c);
#pragma unroll
        for (int k = 0; k < kBInstr; ++k) {
          const int q = wave + C::kWaves * k;
          dma16(rb, bv + dma::rows_group(q, L, 0), stage + C::kBOff + 8 * q * kChunk);
        }
      }
      // scale rows: all 64 lanes (no divergence); lanes past the tile's rows read zeros
      if (wave == 0)
        dma16(make_rsrc(sA + c * I + i0, imin64(I - i0, C::BM) * 4), 16 * lane,
              stage + C::kSAOff);
      if (C::kPerColScale && wave == (1 % C::kWaves))
        dma16(make_rsrc(sB + c * J + j0, imin64(J - j0, C::BN) * 4), 16 * lane,
              stage + C::kSBOff);
    }
  }

  // Second part of chunk c's DMA in an 8-wave block: the issuing half's B rows.
  __device__ __forceinline__ void issue_second(lds_u8* stage, int64_t c) const {
    if constexpr (kPingPong) {
      if (wave / kIssuers == static_cast<int>(c & 1)) issue_as_b(stage, c, wave % kIssuers);
    }
  }

  // The share of issuing wave w (of kIssuers) in an 8-wave block: the A rows with the scale rows,
  // and the B rows.
  __device__ __forceinline__ void issue_as_a(lds_u8* stage, int64_t c, int w) const {
    if (a_inside) {
#pragma unroll
      for (int k = 0; k < kAInstr; ++k) {
        const int q = w + kIssuers * k;
        dma16(ra, a_voff, stage + C::kAOff + 8 * q * kChunk, dma::rows_group(q, L, c));
      }
    } else {
      const uint32_t av = chunk_lane_offset(a_voff, c);
#pragma unroll
      for (int k = 0; k < kAInstr; ++k) {
        const int q = w + kIssuers * k;
        dma16(ra, av + dma::rows_group(q, L, 0), stage + C::kAOff + 8 * q * kChunk);
      }
    }
    // scale rows: all 64 lanes (no divergence); lanes past the tile's rows read zeros
    if (w == 0)
      dma16(make_rsrc(sA + c * I + i0, imin64(I - i0, C::BM) * 4), 16 * lane,
            stage + C::kSAOff);
    if (C::kPerColScale && w == 1)
      dma16(make_rsrc(sB + c * J + j0, imin64(J - j0, C::BN) * 4), 16 * lane,
            stage + C::kSBOff);
  }
  __device__ __forceinline__ void issue_as_b(lds_u8* stage, int64_t c, int w) const {
    if (C::kBTrans) {
      // staged B = BN/128 slabs of 128 reduction rows x 128 columns; slab s holds columns
      // j0 + 128 s .. +127 and its row rr is reduction row rr of the chunk
      const uint8_t* base = B + c * kChunk * J + j0;
      const rsrc_t rbc = make_rsrc(base, (L - c * kChunk) * J - j0);
#pragma unroll
      for (int k = 0; k < kBInstr; ++k) {
        const int q = w + kIssuers * k;
        dma16(rbc, bt_voff[k], stage + C::kBOff + 8 * q * kChunk);
      }
    } else if (b_inside) {
#pragma unroll
      for (int k = 0; k < kBInstr; ++k) {
        const int q = w + kIssuers * k;
        dma16(rb, b_voff, stage + C::kBOff + 8 * q * kChunk, dma::rows_group(q, L, c));
      }
    } else {
      const uint32_t bv = chunk_lane_offset(b_voff, c);
#pragma unroll
      for (int k = 0; k < kBInstr; ++k) {
        const int q = w + kIssuers * k;
        dma16(rb, bv + dma::rows_group(q, L, 0), stage + C::kBOff + 8 * q * kChunk);
      }
    }
  }

};

// Per-lane LDS byte offsets of this wave's fragment reads, fixed for the whole kernel. Every
// row-major fragment covers 16 staged rows starting at a multiple of 16, so its swizzle term
// swz_rows(R0 + r) = swz_rows(r) depends on the lane only; every transposed read of lane
// 16G + r touches slab row 32G + 8i + r/2, whose swz_slab term is the same for all i (row bits
// 3-4 do not enter it).
template <class C>
struct FragOffsets {
  int a[2];    // [half]: A rows, wave-relative
  int b[2];    // same for row-major B
  int bt[4];   // reduction-major B, per nj
  int sa;      // this lane's A scale (row r of each 16-row block)
  int sb;      // this lane's 4 B scales (columns 4G..4G+3 of each 16-column block)
  int sbr;     // power-of-two mode: this lane's B scale (column r of each 16-column block)

  __device__ __forceinline__ void init(int wm, int wn, int lane) {
    const int G = lane >> 4, r = lane & 15;
    for (int e = 0; e < 2; ++e) {
      const int x = ((2 * G + e) ^ swz_rows(r)) << 4;
      a[e] = C::kAOff + (wm * C::WM + r) * kChunk + x;
      b[e] = C::kBOff + (wn * C::WN + r) * kChunk + x;
    }
    // Reduction-major B (dgrad): fragment (nj, i) reads slab (col >> 7), row 32G + 8i + r/2,
    // 8 bytes at 8 * (r & 1) of piece (col & 127) >> 4, where col = wn * WN + 16 nj.
    const int slab = ((wn * C::WN) >> 7) * kSlab;
    const int xs = swz_slab(32 * G + (r >> 1));
    for (int nj = 0; nj < 4; ++nj) {
      const int piece = (((wn * C::WN) & 127) >> 4) + nj;
      bt[nj] = C::kBOff + slab + (32 * G + (r >> 1)) * kChunk + 8 * (r & 1) + ((piece ^ xs) << 4);
    }
    sa = C::kSAOff + (wm * C::WM + r) * 4;
    sb = C::kSBOff + (wn * C::WN + 4 * G) * 4;
    sbr = C::kSBOff + (wn * C::WN + r) * 4;
  }
};

template <int kOff>
__device__ __forceinline__ v4i lds_v4i(const lds_u8* stage, int off) {
  return *reinterpret_cast<const lds_v4i_t*>(stage + off + kOff);
}

// A-type fragment: 16 rows starting at wave row 16*mi.
template <class C, int mi>
__device__ __forceinline__ v8i frag_a(const lds_u8* stage, const FragOffsets<C>& o) {
  const v4i lo = lds_v4i<16 * mi * kChunk>(stage, o.a[0]);
  const v4i hi = lds_v4i<16 * mi * kChunk>(stage, o.a[1]);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <class C, int nj>
__device__ __forceinline__ v8i frag_b(const lds_u8* stage, const FragOffsets<C>& o) {
  if (C::kBTrans) {
    v8i f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_v2i*)(stage + o.bt[nj] + 8 * i * kChunk));
      f[2 * i] = v[0];
      f[2 * i + 1] = v[1];
    }
    return f;
  } else {
    const v4i lo = lds_v4i<16 * nj * kChunk>(stage, o.b[0]);
    const v4i hi = lds_v4i<16 * nj * kChunk>(stage, o.b[1]);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

template <class C, int mi>
__device__ __forceinline__ float scale_a(const lds_u8* stage, const FragOffsets<C>& o) {
  return *reinterpret_cast<const lds_f32*>(stage + o.sa + 16 * mi * 4);
}

// Each MFMA takes the B fragment as its row operand and the A fragment as its column operand,
// so it produces the 16x16 block of C transposed: lane (G, r) receives C row r, columns
// 4G..4G+3. A lane then needs one A scale per 16-row block and, in per-column mode, four B
// scales per 16-column block, and its four results are adjacent in memory.
//
// Software pipeline over the MI x NJ MFMA tiles of a chunk, flattened as k = mi * NJ + nj:
// step k issues MFMA k and then promotes MFMA k - NJ (same column, previous row block), whose
// result is ready by then, so the promotion FMAs run on the vector ALU while the matrix core
// works through the next products. Only NJ + 1 product vectors are live at once. The next row
// block's A fragment and scale are fetched from LDS at the start of each row block.
template <class C>
struct ChunkState {
  static constexpr int kWin = C::NJ + 1;
  using SB = typename std::conditional<C::kPerColScale, v4f, float>::type;
  v8i bf[C::NJ];
  SB sbv[C::NJ];
  v4f p[kWin];
  v8i af_cur, af_next;
  float sa_cur, sa_next, sa_prev;
};

// Hook a chunk runs before its second row block (the second part of the next chunk's DMA in
// 8-wave tiles); by default nothing.
struct NoMid {
  __device__ __forceinline__ void operator()() const {}
};

template <class C, int k, class Mid>
__device__ __forceinline__ void chunk_step(const lds_u8* stage, const FragOffsets<C>& o,
                                           ChunkState<C>& st, float sb_blk,
                                           v4f (&acc)[C::MI][C::NJ], const Mid& mid) {
  constexpr int kTiles = C::MI * C::NJ;
  if constexpr (k < kTiles + C::NJ) {
    constexpr int mi = k / C::NJ, nj = k % C::NJ;
    constexpr int kWin = ChunkState<C>::kWin;
    if constexpr (k < kTiles) {
      if constexpr (nj == 0 && mi + 1 < C::MI) {
        st.af_next = frag_a<C, mi + 1>(stage, o);
        st.sa_next = scale_a<C, mi + 1>(stage, o);
      }
      if constexpr (k == C::NJ) mid();
      st.p[k % kWin] = mfma_fp8(st.bf[nj], st.af_cur);
    }
    if constexpr (k >= C::NJ) {
      constexpr int kp = k - C::NJ;
      constexpr int mp = kp / C::NJ, np = kp % C::NJ;
      if constexpr (C::kPerColScale)
        acc[mp][np] += (st.sa_prev * st.sbv[np]) * st.p[kp % kWin];
      else
        acc[mp][np] += (st.sa_prev * sb_blk) * st.p[kp % kWin];
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
    chunk_step<C, k + 1>(stage, o, st, sb_blk, acc, mid);
  }
}

// The chunk's B fragments, issued in column order, each fence keeping that order: LDS reads
// return in order, so the first product waits only for the first A and B fragments, not for
// the whole chunk's reads.
template <class C, int nj>
__device__ __forceinline__ void load_bf(const lds_u8* stage, const FragOffsets<C>& o,
                                        ChunkState<C>& st, float sb_blk) {
  if constexpr (nj < C::NJ) {
    st.bf[nj] = frag_b<C, nj>(stage, o);
    if constexpr (C::kPerColScale)
      st.sbv[nj] = *reinterpret_cast<const lds_v4f*>(stage + o.sb + 64 * nj);
    else
      st.sbv[nj] = sb_blk;
    __builtin_amdgcn_sched_barrier(0);
    load_bf<C, nj + 1>(stage, o, st, sb_blk);
  }
}

// One 128-wide reduction chunk out of a landed stage: the first A fragment is read first, then
// the B fragments in the order the first row block multiplies them.
template <class C, class Mid = NoMid>
__device__ __forceinline__ void compute_chunk(const lds_u8* stage, float sb_blk,
                                              const FragOffsets<C>& o,
                                              v4f (&acc)[C::MI][C::NJ], const Mid& mid = Mid()) {
  ChunkState<C> st;
  st.af_cur = frag_a<C, 0>(stage, o);
  st.sa_cur = scale_a<C, 0>(stage, o);
  __builtin_amdgcn_sched_barrier(0);
  load_bf<C, 0>(stage, o, st, sb_blk);
  chunk_step<C, 0>(stage, o, st, sb_blk, acc, mid);
}

// ------------------------------------------------------------------ power-of-two scales
// When every scale is a power of two, the matrix core applies them itself: the scaled FP8
// instruction takes one 8-bit biased exponent (E8M0) per operand row and lane, multiplies each
// 32-element reduction block of that row by it, and adds into the accumulator it is given. A
// lane (G, r) supplies the scale of row r of its operand for reduction block G; since one scale
// covers all 128 elements of a chunk, that is simply the scale of row r. The chunk's MI x NJ
// instructions then accumulate straight into acc, with no promotion on the vector ALU.
//
// The E8M0 byte of a positive power-of-two fp32 scale is its exponent field, including
// 2^-127 (fp32 subnormal 0x00400000, field 0, which E8M0 code 0 denotes).
__device__ __forceinline__ int e8m0(float s) { return static_cast<int>(__float_as_uint(s) >> 23); }

template <class C>
struct Pow2State {
  v8i bf[C::NJ];
  int eb[C::NJ];
  v8i af_cur, af_next;
  int ea_cur, ea_next;
};

template <class C, int nj>
__device__ __forceinline__ void load_bf_pow2(const lds_u8* stage, const FragOffsets<C>& o,
                                             Pow2State<C>& st, int eb_blk) {
  if constexpr (nj < C::NJ) {
    st.bf[nj] = frag_b<C, nj>(stage, o);
    if constexpr (C::kPerColScale)
      st.eb[nj] = e8m0(*reinterpret_cast<const lds_f32*>(stage + o.sbr + 64 * nj));
    else
      st.eb[nj] = eb_blk;
    __builtin_amdgcn_sched_barrier(0);
    load_bf_pow2<C, nj + 1>(stage, o, st, eb_blk);
  }
}

// Tile k = mi * NJ + nj; the next row block's A fragment and scale are fetched at the start of
// each row block, as in the promoted path.
template <class C, int k, class Mid>
__device__ __forceinline__ void pow2_step(const lds_u8* stage, const FragOffsets<C>& o,
                                          Pow2State<C>& st, v4f (&acc)[C::MI][C::NJ],
                                          const Mid& mid) {
  if constexpr (k < C::MI * C::NJ) {
    constexpr int mi = k / C::NJ, nj = k % C::NJ;
    if constexpr (nj == 0 && mi + 1 < C::MI) {
      st.af_next = frag_a<C, mi + 1>(stage, o);
      st.ea_next = e8m0(scale_a<C, mi + 1>(stage, o));
    }
    if constexpr (k == C::NJ) mid();
    acc[mi][nj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        st.bf[nj], st.af_cur, acc[mi][nj], 0, 0, 0, st.eb[nj], 0, st.ea_cur);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (nj == C::NJ - 1 && mi + 1 < C::MI) {
      st.af_cur = st.af_next;
      st.ea_cur = st.ea_next;
    }
    pow2_step<C, k + 1>(stage, o, st, acc, mid);
  }
}

template <class C, class Mid = NoMid>
__device__ __forceinline__ void compute_chunk_pow2(const lds_u8* stage, float sb_blk,
                                                   const FragOffsets<C>& o,
                                                   v4f (&acc)[C::MI][C::NJ],
                                                   const Mid& mid = Mid()) {
  Pow2State<C> st;
  st.af_cur = frag_a<C, 0>(stage, o);
  st.ea_cur = e8m0(scale_a<C, 0>(stage, o));
  __builtin_amdgcn_sched_barrier(0);
  load_bf_pow2<C, 0>(stage, o, st, e8m0(sb_blk));
  pow2_step<C, 0>(stage, o, st, acc, mid);
  // Pin the accumulators at the end of the chunk: without this, IR-level sinking moves the
  // chunk's instructions past the next barrier, keeping all its fragments live (spills).
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj) asm volatile("" : "+v"(acc[mi][nj]));
}

// Tile origin of this block. Workgroups are dealt round-robin to the 8 XCDs, so the block id is
// first remapped so that consecutive tiles run on one XCD; tiles are then walked in bands of
// band_rows tile-rows, column by column.
template <class C>
__device__ __forceinline__ void tile_origin(int64_t I, int64_t J, int64_t& i0, int64_t& j0) {
  const int64_t tiles_i = (I + C::BM - 1) / C::BM;
  const int64_t tiles_j = (J + C::BN - 1) / C::BN;
  const int64_t nwg = tiles_i * tiles_j;
  int64_t b = blockIdx.x;
  if ((nwg & 7) == 0) b = (b & 7) * (nwg >> 3) + (b >> 3);
  const int64_t grp = band_rows<C::mode, C::BM>(tiles_j);
  const int64_t band = b / (grp * tiles_j);
  const int64_t rows = imin64(grp, tiles_i - band * grp);
  const int64_t local = b - band * grp * tiles_j;
  const int64_t ti = band * grp + local % rows;
  const int64_t tj = local / rows;
  i0 = uniform64(ti * C::BM);
  j0 = uniform64(tj * C::BN);
}

// Epilogue: lane (G, r) holds row r, columns 4G..4G+3 of every 16x16 block: one 8-byte (bf16)
// or 16-byte (fp32) store per block.
template <class C>
__device__ __forceinline__ void store_tile(const v4f (&acc)[C::MI][C::NJ], void* Cout, int64_t I,
                                           int64_t J, int64_t i0, int64_t j0, int wm, int wn,
                                           int lane, int accumulate) {
  const int G = lane >> 4, r16 = lane & 15;
  const int64_t r0 = i0 + wm * C::WM, q0 = j0 + wn * C::WN;
  if (r0 >= I || q0 >= J) return;  // this wave lies in the invalid half of an edge tile
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) {
#pragma unroll
    for (int nj = 0; nj < C::NJ; ++nj) {
      const int64_t row = r0 + 16 * mi + r16;
      const int64_t col = q0 + 16 * nj + 4 * G;
      const v4f v = acc[mi][nj];
      if (C::kOutF32) {
        v4f* out = reinterpret_cast<v4f*>(static_cast<float*>(Cout) + row * J + col);
        *out = accumulate ? *out + v : v;
      } else {
        v2i packed;
        packed[0] = static_cast<int>(pack_bf16x2(v[0], v[1]));
        packed[1] = static_cast<int>(pack_bf16x2(v[2], v[3]));
        *reinterpret_cast<v2i*>(static_cast<uint16_t*>(Cout) + row * J + col) = packed;
      }
    }
  }
}

// Epilogue through LDS, for waves 64 columns wide. Stored straight from the fragments, each
// instruction writes 16 rows x 4 columns, a quarter (bf16) or half (fp32) of a cache line per
// row, and on MI355X the output stores of a round of bf16 tiles took about 9 us, a quarter of a
// 16-chunk tile's time. Instead each wave converts its block into a private LDS region and then
// writes whole rows, 16 bytes per lane, so every store covers full lines (measured: 2-4 us less
// per round of tiles). The regions lie in the stage the last chunk did not use: every wave has
// passed the barrier in front of that chunk, which came after all reads of the other stage, and
// no DMA is issued after it, so no further barrier is needed and each wave starts its stores
// as soon as its own products are done (measured: 0.8 % on a 28-layer linear-stack training step
// against restaging into both stages behind one more barrier). One stage holds every wave's region for a share of its rows,
// so the block goes in 1-6 passes over its rows; the 16-byte units of a row are XOR-swizzled by
// the row's low bits so that the row reads do not conflict on LDS banks.
template <class C>
__device__ __forceinline__ void store_tile_lds(const v4f (&acc)[C::MI][C::NJ], void* Cout,
                                               int64_t I, int64_t J, int64_t i0, int64_t j0,
                                               int wm, int wn, int wave, int lane, int accumulate,
                                               lds_u8* free_stage) {
  constexpr int kElt = C::kOutF32 ? 4 : 2;
  constexpr int kRowBytes = kElt * C::WN;
  constexpr int kUnits = kRowBytes / 16;  // 16-byte units per row: 8 (bf16) or 16 (fp32)
  constexpr int kBlockBytes = C::kWaves * C::WM * kRowBytes;
  constexpr int kPasses = kBlockBytes <= C::kStageBytes                          ? 1
                          : kBlockBytes <= 2 * C::kStageBytes && C::MI % 2 == 0 ? 2
                          : kBlockBytes <= 4 * C::kStageBytes && C::MI % 4 == 0 ? 4
                                                                                : C::MI;
  constexpr int kPassMI = C::MI / kPasses;
  constexpr int kRows = 16 * kPassMI;  // rows of the block per pass
  constexpr int kRowsPerStore = 64 / kUnits;
  static_assert(C::WN == 64 && C::MI % kPasses == 0, "64-column waves, whole fragments a pass");
  static_assert(C::kWaves * kRows * kRowBytes <= C::kStageBytes, "regions fit one stage");
  const int64_t r0 = i0 + wm * C::WM, q0 = j0 + wn * C::WN;
  if (r0 >= I || q0 >= J) return;  // this wave lies in the invalid half of an edge tile
  lds_u8* region = free_stage + wave * kRows * kRowBytes;
  const int G = lane >> 4, r16 = lane & 15;
  const int lr = lane / kUnits, lu = lane % kUnits;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
#pragma unroll
    for (int m = 0; m < kPassMI; ++m) {
      const int row = 16 * m + r16;
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj) {
        const v4f v = acc[pass * kPassMI + m][nj];
        if constexpr (C::kOutF32) {
          const int unit = 4 * nj + G;
          *reinterpret_cast<lds_v4f*>(region + row * kRowBytes + 16 * (unit ^ (row & 7))) = v;
        } else {
          const int unit = 2 * nj + (G >> 1);
          v2i packed;
          packed[0] = static_cast<int>(pack_bf16x2(v[0], v[1]));
          packed[1] = static_cast<int>(pack_bf16x2(v[2], v[3]));
          *reinterpret_cast<lds_v2i*>(region + row * kRowBytes + 16 * (unit ^ (row & 7)) +
                                      8 * (G & 1)) = packed;
        }
      }
    }
    // the reads below take other lanes' writes: wait for them, and keep the compiler from
    // moving any LDS access across
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int p = 0; p < kRows / kRowsPerStore; ++p) {
      const int row = kRowsPerStore * p + lr;
      const v4i raw = *reinterpret_cast<const lds_v4i_t*>(region + row * kRowBytes +
                                                          16 * (lu ^ (row & 7)));
      const int64_t grow = r0 + pass * kRows + row;
      if constexpr (C::kOutF32) {
        v4f* out = reinterpret_cast<v4f*>(static_cast<float*>(Cout) + grow * J + q0 + 4 * lu);
        const v4f v = __builtin_bit_cast(v4f, raw);
        *out = accumulate ? *out + v : v;
      } else {
        // Non-temporal: Y and dX are next read by other operations, later; keeping them out of
        // L2 and the memory-side cache leaves room for the operands and codes that the GEMMs and
        // quantisers in between do read (measured on a 28-layer linear-stack training step:
        // 39.9 -> 39.3 ms, the quantisers 3-7 % faster).
        __builtin_nontemporal_store(
            raw, reinterpret_cast<v4i*>(static_cast<uint16_t*>(Cout) + grow * J + q0 + 8 * lu));
      }
    }
    // the next pass overwrites the region: keep its writes after these reads
    if (pass + 1 < kPasses) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

template <class C>
__device__ __forceinline__ void gemm_body(const uint8_t* __restrict__ A,
                                          const float* __restrict__ sA,
                                          const uint8_t* __restrict__ B,
                                          const float* __restrict__ sB, void* __restrict__ Cout,
                                          int64_t I, int64_t J, int64_t L, int accumulate,
                                          lds_u8* stage0, lds_u8* stage1) {
  int64_t i0, j0;
  tile_origin<C>(I, J, i0, j0);

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

  if (nk > 0) {
    ld.issue(stage0, 0);
    ld.issue_second(stage0, 0);
  }
  float sb_next = (!C::kPerColScale && nk > 0) ? ld.sb_block[0] : 0.0f;

  // Chunks go in pairs (stage0 then stage1) so that each stage is a distinct LDS object; an odd
  // last chunk is handled after the loop. Every half: wait for this wave's DMA, barrier (the
  // stage has landed for all waves, and the other stage is no longer being read), enqueue the
  // next chunk into the other stage, multiply out of this one.
  auto half = [&](lds_u8* cur, lds_u8* nxt, int64_t c) {
    const float sb = sb_next;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (c + 1 < nk) {
      ld.issue(nxt, c + 1);
      if (!C::kPerColScale) sb_next = ld.block_scale(c + 1);
    }
    auto mid = [&]() {  // runs before the chunk's second row block
      if (c + 1 < nk) ld.issue_second(nxt, c + 1);
    };
    if constexpr (C::kPow2)
      compute_chunk_pow2<C>(cur, sb, fo, acc, mid);
    else
      compute_chunk<C>(cur, sb, fo, acc, mid);
  };
  int64_t c = 0;
  for (; c + 1 < nk; c += 2) {
    half(stage0, stage1, c);
    half(stage1, stage0, c + 1);
  }
  if (c < nk) half(stage0, stage1, c);

  if constexpr (C::WN == 64)
    store_tile_lds<C>(acc, Cout, I, J, i0, j0, wm, wn, wave, lane, accumulate,
                      (nk & 1) ? stage1 : stage0);
  else
    store_tile<C>(acc, Cout, I, J, i0, j0, wm, wn, lane, accumulate);
}

// Weight gradient of a small output with the reduction split inside the block: two groups of
// the configuration's waves share one BM x BN tile, group g multiplying out chunks g, g+2, g+4,
// ... from stages of its own, so a 128 x 128 tile gets 8 waves (two per SIMD) instead of 4.
// At the end group 1 hands its partial sums to group 0 through LDS, which adds them (fixed
// order, so the result is deterministic) and stores the tile.
constexpr int kRedPitch = 132;  // floats per row of the reduction buffer

template <class C>
__device__ __forceinline__ void gemm_body_k2(const uint8_t* __restrict__ A,
                                             const float* __restrict__ sA,
                                             const uint8_t* __restrict__ B,
                                             const float* __restrict__ sB, void* __restrict__ Cout,
                                             int64_t I, int64_t J, int64_t L, int accumulate,
                                             lds_u8* stage0, lds_u8* stage1) {
  static_assert(C::mode == kWgrad, "split reduction is a weight-gradient shape");
  static_assert(C::BM * kRedPitch * 4 <= 2 * C::kStageBytes, "reduction buffer fits a stage pair");
  int64_t i0, j0;
  tile_origin<C>(I, J, i0, j0);
  const int t = threadIdx.x;
  const int wave_all = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = wave_all / C::kWaves;  // reduction group
  const int wave = wave_all % C::kWaves;
  const int lane = t & 63;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int64_t nk = L / kChunk;

  Loader<C, false> ld;  // the scalar-offset form spills here (see Loader)
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

  // group g's stages: [g * kStageBytes, (g + 1) * kStageBytes) of each stage object
  const int goff = g * C::kStageBytes;
  if (g < nk) ld.issue(stage0 + goff, g);
  auto half = [&](lds_u8* cur, lds_u8* nxt, int64_t p) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int64_t cn = 2 * (p + 1) + g;
    // group 0 issues its next chunk right away, group 1 before its second row block, so that
    // the two waves sharing a SIMD do not both feed the memory pipeline at once
    if (g == 0 && cn < nk) ld.issue(nxt + goff, cn);
    auto mid = [&]() {
      if (g == 1 && cn < nk) ld.issue(nxt + goff, cn);
    };
    if (2 * p + g < nk) {
      if constexpr (C::kPow2)
        compute_chunk_pow2<C>(cur + goff, 0.0f, fo, acc, mid);
      else
        compute_chunk<C>(cur + goff, 0.0f, fo, acc, mid);
    } else {
      mid();
    }
  };
  const int64_t steps = (nk + 1) / 2;
  int64_t p = 0;
  for (; p + 1 < steps; p += 2) {
    half(stage0, stage1, p);
    half(stage1, stage0, p + 1);
  }
  if (p < steps) half(stage0, stage1, p);

  // reduction through LDS (both stage objects are free once every wave has passed this barrier)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int G = lane >> 4, r16 = lane & 15;
  lds_f32* red = reinterpret_cast<lds_f32*>(stage0);
  if (g == 1) {
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj)
        *reinterpret_cast<lds_v4f*>(red + (wm * C::WM + 16 * mi + r16) * kRedPitch +
                                    wn * C::WN + 16 * nj + 4 * G) = acc[mi][nj];
  }
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int nj = 0; nj < C::NJ; ++nj)
        acc[mi][nj] += *reinterpret_cast<const lds_v4f*>(
            red + (wm * C::WM + 16 * mi + r16) * kRedPitch + wn * C::WN + 16 * nj + 4 * G);
    store_tile<C>(acc, Cout, I, J, i0, j0, wm, wn, lane, accumulate);
  }
}

// Two tile shapes: 256x256 (8 waves of 128x64, one block per CU) for GEMMs with at least one
// full wave of such tiles, and 128x128 (4 waves of 64x64, two blocks per CU) for GEMMs whose
// output is too small to fill the chip with big tiles (e.g. the weight gradients of the
// 2048-wide projections).
using FwdBig = Cfg<kFwd, 256, 256, 2, 4>;
using DgradBig = Cfg<kDgrad, 256, 256, 2, 4>;
using WgradBig = Cfg<kWgrad, 256, 256, 2, 4>;
using FwdSmall = Cfg<kFwd, 128, 128, 2, 2>;
using DgradSmall = Cfg<kDgrad, 128, 128, 2, 2>;
using WgradSmall = Cfg<kWgrad, 128, 128, 2, 2>;
// Extra weight-gradient shapes that make common outputs whole rounds of tiles: 256x192 (8 waves
// of 128x48; a 2048 x 6144 output is 256 tiles) and 192x256 (8 waves of 96x64; a 12288 x 2048
// output is 512 tiles).
using WgradWide = Cfg<kWgrad, 256, 192, 2, 4>;
using WgradTall = Cfg<kWgrad, 192, 256, 2, 4>;
// The same shapes with power-of-two scales.
using FwdBigP2 = Cfg<kFwd, 256, 256, 2, 4, true>;
using DgradBigP2 = Cfg<kDgrad, 256, 256, 2, 4, true>;
using WgradBigP2 = Cfg<kWgrad, 256, 256, 2, 4, true>;
using FwdSmallP2 = Cfg<kFwd, 128, 128, 2, 2, true>;
using DgradSmallP2 = Cfg<kDgrad, 128, 128, 2, 2, true>;
using WgradSmallP2 = Cfg<kWgrad, 128, 128, 2, 2, true>;
using WgradWideP2 = Cfg<kWgrad, 256, 192, 2, 4, true>;
using WgradTallP2 = Cfg<kWgrad, 192, 256, 2, 4, true>;

#define PURO_GEMM_KERNEL(NAME, CFG)                                                        \
  __global__ __launch_bounds__(CFG::kThreads) void NAME(                                   \
      const uint8_t* __restrict__ A, const float* __restrict__ sA,                         \
      const uint8_t* __restrict__ B, const float* __restrict__ sB, void* __restrict__ Cout, \
      int64_t I, int64_t J, int64_t L, int accumulate) {                                   \
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[CFG::kStageBytes];            \
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[CFG::kStageBytes];            \
    gemm_body<CFG>(A, sA, B, sB, Cout, I, J, L, accumulate, (lds_u8*)stage0,               \
                   (lds_u8*)stage1);                                                        \
  }

PURO_GEMM_KERNEL(gemm_fwd_256x256, FwdBig)
PURO_GEMM_KERNEL(gemm_dgrad_256x256, DgradBig)
PURO_GEMM_KERNEL(gemm_wgrad_256x256, WgradBig)
PURO_GEMM_KERNEL(gemm_fwd_128x128, FwdSmall)
PURO_GEMM_KERNEL(gemm_dgrad_128x128, DgradSmall)
PURO_GEMM_KERNEL(gemm_wgrad_128x128, WgradSmall)
PURO_GEMM_KERNEL(gemm_wgrad_256x192, WgradWide)
PURO_GEMM_KERNEL(gemm_wgrad_192x256, WgradTall)
PURO_GEMM_KERNEL(gemm_fwd_256x256_pow2, FwdBigP2)
PURO_GEMM_KERNEL(gemm_dgrad_256x256_pow2, DgradBigP2)
PURO_GEMM_KERNEL(gemm_wgrad_256x256_pow2, WgradBigP2)
PURO_GEMM_KERNEL(gemm_fwd_128x128_pow2, FwdSmallP2)
PURO_GEMM_KERNEL(gemm_dgrad_128x128_pow2, DgradSmallP2)
PURO_GEMM_KERNEL(gemm_wgrad_128x128_pow2, WgradSmallP2)
PURO_GEMM_KERNEL(gemm_wgrad_256x192_pow2, WgradWideP2)
PURO_GEMM_KERNEL(gemm_wgrad_192x256_pow2, WgradTallP2)

#define PURO_GEMM_KERNEL_K2(NAME, CFG)                                                     \
  __global__ __launch_bounds__(2 * CFG::kThreads) void NAME(                               \
      const uint8_t* __restrict__ A, const float* __restrict__ sA,                         \
      const uint8_t* __restrict__ B, const float* __restrict__ sB, void* __restrict__ Cout, \
      int64_t I, int64_t J, int64_t L, int accumulate) {                                   \
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[2 * CFG::kStageBytes];        \
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[2 * CFG::kStageBytes];        \
    gemm_body_k2<CFG>(A, sA, B, sB, Cout, I, J, L, accumulate, (lds_u8*)stage0,            \
                      (lds_u8*)stage1);                                                     \
  }

PURO_GEMM_KERNEL_K2(gemm_wgrad_128x128_k2, WgradSmall)
PURO_GEMM_KERNEL_K2(gemm_wgrad_128x128_k2_pow2, WgradSmallP2)

// Number of compute units the big tiles must at least fill once.
constexpr int64_t kComputeUnits = 256;

inline bool use_big_tiles(int64_t I, int64_t J) {
  return ((I + 255) / 256) * ((J + 255) / 256) >= kComputeUnits;
}

// Compute units of the current device.
inline int64_t device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return kComputeUnits;
  return cus;
}

// Weight-gradient tile shape: the candidate with the least estimated time, counting whole
// rounds of tiles over the chip (a partial last round costs a full one), each tile's area,
// the blocks resident per CU (LDS and registers allow one 8-wave block of the 256-row shapes,
// two 4-wave 128x128 blocks, or one 8-wave split-reduction 128x128 block), and a per-shape
// efficiency measured on MI355X (bigger tiles re-read less). The 192- and 256-wide shapes are
// only used when they tile the output exactly. The split-reduction figure sits between its two
// measured cases: on a 2048 x 2048 output (one tile per CU) it beats the four-wave blocks by
// 10-15 %, on a 4096 x 2048 output (two rounds against one round of two blocks per CU) it
// loses by 25 %.
enum WgradShape { kW256x256, kW128x128, kW256x192, kW192x256, kW128x128k2 };

inline WgradShape pick_wgrad_shape(int64_t I, int64_t J) {
  struct Cand {
    WgradShape shape;
    int64_t bm, bn, resident;
    double eff;
    bool exact_only;
  };
  const Cand cands[] = {
      {kW256x256, 256, 256, 1, 1.00, true},
      {kW128x128, 128, 128, 2, 0.85, false},
      {kW128x128k2, 128, 128, 1, 0.60, false},
      {kW256x192, 256, 192, 1, 0.97, true},
      {kW192x256, 192, 256, 1, 0.97, true},
  };
  const int64_t cus = device_cus();
  WgradShape best = kW256x256;
  double best_cost = -1.0;
  for (const Cand& c : cands) {
    if (c.exact_only && (I % c.bm != 0 || J % c.bn != 0)) continue;
    const int64_t tiles = ((I + c.bm - 1) / c.bm) * ((J + c.bn - 1) / c.bn);
    const int64_t slots = cus * c.resident;
    const int64_t rounds = (tiles + slots - 1) / slots;
    const double cost = static_cast<double>(rounds) * c.bm * c.bn * c.resident / c.eff;
    if (best_cost < 0.0 || cost < best_cost) {
      best_cost = cost;
      best = c.shape;
    }
  }
  return best;
}

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

template <class C>
puro_status launch_k2(GemmKernel k, const void* A, const float* sA, const void* B,
                      const float* sB, void* Cout, int64_t I, int64_t J, int64_t L,
                      int accumulate, void* stream) {
  const int64_t blocks = ((I + C::BM - 1) / C::BM) * ((J + C::BN - 1) / C::BN);
  if (blocks > INT32_MAX) return PURO_ERR_SHAPE;
  hipLaunchKernelGGL(k, dim3(static_cast<uint32_t>(blocks)), dim3(2 * C::kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(A), sA,
                     static_cast<const uint8_t*>(B), sB, Cout, I, J, L, accumulate);
  return launch_status();
}

// Kernels of one scale rule.
template <bool kPow2>
struct Kernels;
template <>
struct Kernels<false> {
  using FwdB = FwdBig;
  using FwdS = FwdSmall;
  using DgB = DgradBig;
  using DgS = DgradSmall;
  using WgB = WgradBig;
  using WgS = WgradSmall;
  using WgW = WgradWide;
  using WgT = WgradTall;
  static constexpr GemmKernel fwd_b = gemm_fwd_256x256, fwd_s = gemm_fwd_128x128;
  static constexpr GemmKernel dg_b = gemm_dgrad_256x256, dg_s = gemm_dgrad_128x128;
  static constexpr GemmKernel wg_b = gemm_wgrad_256x256, wg_s = gemm_wgrad_128x128;
  static constexpr GemmKernel wg_w = gemm_wgrad_256x192, wg_t = gemm_wgrad_192x256;
  static constexpr GemmKernel wg_k2 = gemm_wgrad_128x128_k2;
};
template <>
struct Kernels<true> {
  using FwdB = FwdBigP2;
  using FwdS = FwdSmallP2;
  using DgB = DgradBigP2;
  using DgS = DgradSmallP2;
  using WgB = WgradBigP2;
  using WgS = WgradSmallP2;
  using WgW = WgradWideP2;
  using WgT = WgradTallP2;
  static constexpr GemmKernel fwd_b = gemm_fwd_256x256_pow2, fwd_s = gemm_fwd_128x128_pow2;
  static constexpr GemmKernel dg_b = gemm_dgrad_256x256_pow2, dg_s = gemm_dgrad_128x128_pow2;
  static constexpr GemmKernel wg_b = gemm_wgrad_256x256_pow2, wg_s = gemm_wgrad_128x128_pow2;
  static constexpr GemmKernel wg_w = gemm_wgrad_256x192_pow2, wg_t = gemm_wgrad_192x256_pow2;
  static constexpr GemmKernel wg_k2 = gemm_wgrad_128x128_k2_pow2;
};

template <bool kPow2>
puro_status gemm_fwd(const void* xq, const float* sx, const void* wq, const float* sw, void* y,
                     int64_t M, int64_t N, int64_t K, void* stream) {
  using Ks = Kernels<kPow2>;
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K)) return PURO_ERR_SHAPE;
  const bool out_empty = M == 0 || N == 0;
  const bool red_empty = out_empty || K == 0;
  PURO_TRY(check_ptr(xq, red_empty));
  PURO_TRY(check_ptr(sx, red_empty));
  PURO_TRY(check_ptr(wq, red_empty));
  PURO_TRY(check_ptr(sw, red_empty));
  PURO_TRY(check_ptr(y, out_empty));
  if (out_empty) return PURO_OK;
  PURO_TRY(debug::check_operand(xq, M * K, sx, (K / 128) * M, stream));
  PURO_TRY(debug::check_operand(wq, N * K, sw, (N / 128) * (K / 128), stream));
  if (use_big_tiles(M, N))
    return launch<typename Ks::FwdB>(Ks::fwd_b, xq, sx, wq, sw, y, M, N, K, 0, stream);
  return launch<typename Ks::FwdS>(Ks::fwd_s, xq, sx, wq, sw, y, M, N, K, 0, stream);
}

template <bool kPow2>
puro_status gemm_dgrad(const void* dyq, const float* sdy, const void* wq, const float* sw,
                       void* dx, int64_t M, int64_t N, int64_t K, void* stream) {
  using Ks = Kernels<kPow2>;
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K)) return PURO_ERR_SHAPE;
  const bool out_empty = M == 0 || K == 0;
  const bool red_empty = out_empty || N == 0;
  PURO_TRY(check_ptr(dyq, red_empty));
  PURO_TRY(check_ptr(sdy, red_empty));
  PURO_TRY(check_ptr(wq, red_empty));
  PURO_TRY(check_ptr(sw, red_empty));
  PURO_TRY(check_ptr(dx, out_empty));
  if (out_empty) return PURO_OK;
  PURO_TRY(debug::check_operand(dyq, M * N, sdy, (N / 128) * M, stream));
  PURO_TRY(debug::check_operand(wq, N * K, sw, (N / 128) * (K / 128), stream));
  if (use_big_tiles(M, K))
    return launch<typename Ks::DgB>(Ks::dg_b, dyq, sdy, wq, sw, dx, M, K, N, 0, stream);
  return launch<typename Ks::DgS>(Ks::dg_s, dyq, sdy, wq, sw, dx, M, K, N, 0, stream);
}

template <bool kPow2>
puro_status gemm_wgrad(const void* dytq, const float* sdyt, const void* xtq, const float* sxt,
                       float* dw, int64_t M, int64_t N, int64_t K, int accumulate,
                       void* stream) {
  using Ks = Kernels<kPow2>;
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
  PURO_TRY(debug::check_operand(dytq, N * M, sdyt, (M / 128) * N, stream));
  PURO_TRY(debug::check_operand(xtq, K * M, sxt, (M / 128) * K, stream));
  switch (pick_wgrad_shape(N, K)) {
    case kW256x256:
      return launch<typename Ks::WgB>(Ks::wg_b, dytq, sdyt, xtq, sxt, dw, N, K, M, accumulate,
                                      stream);
    case kW256x192:
      return launch<typename Ks::WgW>(Ks::wg_w, dytq, sdyt, xtq, sxt, dw, N, K, M, accumulate,
                                      stream);
    case kW192x256:
      return launch<typename Ks::WgT>(Ks::wg_t, dytq, sdyt, xtq, sxt, dw, N, K, M, accumulate,
                                      stream);
    case kW128x128k2:
      return launch_k2<typename Ks::WgS>(Ks::wg_k2, dytq, sdyt, xtq, sxt, dw, N, K, M,
                                         accumulate, stream);
    default:
      return launch<typename Ks::WgS>(Ks::wg_s, dytq, sdyt, xtq, sxt, dw, N, K, M, accumulate,
                                      stream);
  }
}

}  // namespace
}  // namespace puro

using namespace puro;

extern "C" puro_status puro_fp8_gemm_fwd(const void* xq, const float* sx, const void* wq,
                                         const float* sw, void* y, int64_t M, int64_t N,
                                         int64_t K, void* stream) {
  return gemm_fwd<false>(xq, sx, wq, sw, y, M, N, K, stream);
}
extern "C" puro_status puro_fp8_gemm_dgrad(const void* dyq, const float* sdy, const void* wq,
                                           const float* sw, void* dx, int64_t M, int64_t N,
                                           int64_t K, void* stream) {
  return gemm_dgrad<false>(dyq, sdy, wq, sw, dx, M, N, K, stream);
}
extern "C" puro_status puro_fp8_gemm_wgrad(const void* dytq, const float* sdyt, const void* xtq,
                                           const float* sxt, float* dw, int64_t M, int64_t N,
                                           int64_t K, int accumulate, void* stream) {
  return gemm_wgrad<false>(dytq, sdyt, xtq, sxt, dw, M, N, K, accumulate, stream);
}

extern "C" puro_status puro_fp8_gemm_fwd_pow2(const void* xq, const float* sx, const void* wq,
                                              const float* sw, void* y, int64_t M, int64_t N,
                                              int64_t K, void* stream) {
  return gemm_fwd<true>(xq, sx, wq, sw, y, M, N, K, stream);
}
extern "C" puro_status puro_fp8_gemm_dgrad_pow2(const void* dyq, const float* sdy, const void* wq,
                                                const float* sw, void* dx, int64_t M, int64_t N,
                                                int64_t K, void* stream) {
  return gemm_dgrad<true>(dyq, sdy, wq, sw, dx, M, N, K, stream);
}
extern "C" puro_status puro_fp8_gemm_wgrad_pow2(const void* dytq, const float* sdyt,
                                                const void* xtq, const float* sxt, float* dw,
                                                int64_t M, int64_t N, int64_t K, int accumulate,
                                                void* stream) {
  return gemm_wgrad<true>(dytq, sdyt, xtq, sxt, dw, M, N, K, accumulate, stream);
}

// Name of the kernel function a GEMM entry point launches for the given sizes, from the same
// shape choice the entry point makes (for profiling and per-kernel accounting).
extern "C" const char* puro_gemm_kernel_name(int op, int64_t M, int64_t N, int64_t K, int pow2) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || (pow2 != 0 && pow2 != 1)) return nullptr;
  static const char* const kFwd[2][2] = {{"gemm_fwd_128x128", "gemm_fwd_256x256"},
                                         {"gemm_fwd_128x128_pow2", "gemm_fwd_256x256_pow2"}};
  static const char* const kDgrad[2][2] = {
      {"gemm_dgrad_128x128", "gemm_dgrad_256x256"},
      {"gemm_dgrad_128x128_pow2", "gemm_dgrad_256x256_pow2"}};
  switch (op) {
    case 0:
      if (M == 0 || N == 0) return nullptr;
      return kFwd[pow2][use_big_tiles(M, N) ? 1 : 0];
    case 1:
      if (M == 0 || K == 0) return nullptr;
      return kDgrad[pow2][use_big_tiles(M, K) ? 1 : 0];
    case 2: {
      if (N == 0 || K == 0) return nullptr;
      static const char* const kWgrad[2][5] = {
          {"gemm_wgrad_256x256", "gemm_wgrad_128x128", "gemm_wgrad_256x192",
           "gemm_wgrad_192x256", "gemm_wgrad_128x128_k2"},
          {"gemm_wgrad_256x256_pow2", "gemm_wgrad_128x128_pow2", "gemm_wgrad_256x192_pow2",
           "gemm_wgrad_192x256_pow2", "gemm_wgrad_128x128_k2_pow2"}};
      return kWgrad[pow2][pick_wgrad_shape(N, K)];
    }
    default:
      return nullptr;
  }
}

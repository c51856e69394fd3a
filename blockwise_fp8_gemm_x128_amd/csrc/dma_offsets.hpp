// Byte offsets of the GEMM tiles' LDS-DMA loads (buffer_load_dwordx4 ... lds), relative to the
// buffer resource each load goes through. Plain constexpr arithmetic, so the same functions
// serve the kernels and a host-side model of the hardware range check.
//
// A raw buffer load reads zero when its offset lies at or beyond the resource's byte count.
// Whether the scalar offset operand takes part in that check is not something to rely on, so
// every load of a tile that lies partly outside its operand passes its whole offset as the
// per-lane offset (scalar offset 0): the check then covers the row and column the lane
// addresses, and the invalid part of an edge tile reads zeros without touching memory past the
// tensor. Row-major tiles wholly inside their operand address only its own bytes: there the
// lane part (rows_lane) is the per-lane offset and the wave-uniform part (rows_group) the scalar
// one, and no range check is needed.
#pragma once
#include <stdint.h>

namespace puro {
namespace dma {

// Row-major operand (A, and B of the forward and weight-gradient GEMMs): instruction q of a
// chunk stages tile rows [8q, 8q + 8); lane (r8, slot) fetches 16 bytes of row 8q + r8 at byte
// 16 * piece of chunk c, where piece is the logical 16-byte piece of the 128-byte chunk row that
// the lane's LDS slot holds. The resource starts at the tile's first row; its byte count is
// (valid rows) * pitch, so a row at or past the tensor's end fails the check.
constexpr uint32_t rows_lane(int r8, int piece, int64_t pitch) {
  return static_cast<uint32_t>(r8 * pitch + (piece << 4));
}
constexpr uint32_t rows_group(int q, int64_t pitch, int64_t c) {
  return static_cast<uint32_t>(8 * q * pitch + c * 128);
}

// Reduction-major slabs (B of the data-gradient GEMM, W[N][K] read down its columns): staged
// slab sl holds tile columns [128 sl, 128 sl + 128) of one 128-row reduction chunk; instruction
// q (qq = q mod 16, sl = q / 16) stages chunk rows [8 qq, 8 qq + 8) of slab sl, lane (r8, piece)
// the 16 bytes of chunk row 8 qq + r8 at column 128 sl + 16 piece. The resource starts at the
// chunk's first row, tile column 0, and ends at the end of the tensor, so a column past the last
// row's end fails the check (columns past the tensor's width in earlier rows read that row's
// successor: bytes inside the tensor that only feed output columns outside it).
constexpr uint32_t slab_lane(int q, int r8, int piece, int64_t pitch) {
  return static_cast<uint32_t>((8 * (q & 15) + r8) * pitch + 128 * (q >> 4) + (piece << 4));
}

}  // namespace dma
}  // namespace puro

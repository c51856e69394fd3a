// Host-side model of the raw-buffer range check on the GEMM tiles' LDS-DMA loads.
//
// The kernels form every load's offset from the constexpr functions in csrc/dma_offsets.hpp;
// this program calls the same functions, walks the same issue loops (instruction k of issuing
// wave w stages row group q = w + issuers * k; the lane's swizzled piece as in the kernel), and
// checks, for tiles that lie partly outside the tensor:
//   - a row-major load is in range exactly when the row it addresses is inside the tensor, and
//     then it addresses the element the LDS slot expects;
//   - a slab (transposed) load that is in range stays inside the tensor, addresses the expected
//     element when its column is inside the tensor, and the last row's columns past the end are
//     out of range;
//   - a scale-row load is in range exactly when its four scales belong to valid rows.
// The model of the check: a lane's 16 bytes are read when offset < the resource's byte count.
// Edge tiles pass the whole offset per lane (scalar offset 0), so there is no question of
// whether the scalar offset is checked. Row-major tiles that lie wholly inside their operand
// keep the row-group and chunk part in the scalar offset; for them the model checks that every
// lane addresses the expected element inside the tensor and is in range whether the check
// includes the scalar offset or not.
// Prints "ok" and exits 0, or prints the first violations and exits 1.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "dma_offsets.hpp"

using puro::dma::rows_group;
using puro::dma::rows_lane;
using puro::dma::slab_lane;

static int failures = 0;
static void fail(const char* what, long a, long b, long c, long d) {
  if (failures++ < 10) std::printf("FAIL %s: %ld %ld %ld %ld\n", what, a, b, c, d);
}

// swizzles as in the kernels (they only permute pieces inside a 128-byte row)
static int swz_rows(int row) { return ((row & 3) << 1) | ((row >> 3) & 1); }
static int swz_slab(int row) { return ((row >> 1) & 3) | ((row >> 3) & 4); }

static uint32_t records(int64_t bytes) {
  return bytes > int64_t(0xffffffff) ? 0xffffffffu : static_cast<uint32_t>(bytes);
}

// Row-major operand of T rows x L bytes, tiles of `tile` rows, loads issued by `issuers` waves
// with `instr` instructions each (instr * issuers * 8 = tile rows).
static void check_rows(int64_t T, int64_t L, int tile, int issuers) {
  const int instr = tile / 8 / issuers;
  for (int64_t t0 = 0; t0 < T; t0 += tile) {
    const uint32_t nrec = records((T - t0) * L);
    for (int64_t c = 0; c < L / 128; ++c)
      for (int w = 0; w < issuers; ++w)
        for (int k = 0; k < instr; ++k) {
          const int q = w + issuers * k;
          for (int lane = 0; lane < 64; ++lane) {
            const int r8 = lane >> 3, p8 = lane & 7;
            const int xr = swz_rows(8 * w + r8);  // the kernel's per-lane swizzle
            if (xr != swz_rows(8 * q + r8)) fail("row swizzle", q, r8, w, k);
            const int piece = p8 ^ xr;
            const int64_t row = t0 + 8 * q + r8;
            if (T - t0 >= tile) {
              // interior tile: lane part per lane, row group and chunk in the scalar offset
              const uint32_t lv = rows_lane(r8, piece, L), so = rows_group(q, L, c);
              const int64_t addr = t0 * L + int64_t(lv) + int64_t(so);
              if (addr != row * L + c * 128 + 16 * piece) fail("inner address", row, c, piece, addr);
              if (addr < 0 || addr + 16 > T * L) fail("inner past end", T, L, row, addr);
              if (!(lv < nrec) || !(int64_t(lv) + int64_t(so) < int64_t(nrec)))
                fail("inner range", T, L, row, int64_t(lv) + int64_t(so));
              continue;
            }
            const uint32_t voff = rows_lane(r8, piece, L) + rows_group(q, L, 0) +
                                  static_cast<uint32_t>(c * 128);
            const bool in_range = voff < nrec;
            if (in_range != (row < T)) fail("row range", T, L, row, voff);
            if (in_range) {
              const int64_t addr = t0 * L + voff;  // byte address from the tensor's start
              if (addr != row * L + c * 128 + 16 * piece) fail("row address", row, c, piece, addr);
              if (addr + 16 > T * L) fail("row past end", T, L, row, addr);
            }
          }
        }
  }
}

// Data-gradient B: W[L][J] (reduction rows L, tile columns J), slabs of 128 columns.
static void check_slabs(int64_t L, int64_t J, int tile, int issuers) {
  const int instr = tile / 8 / issuers;  // tile/128 slabs x 16 row groups
  for (int64_t j0 = 0; j0 < J; j0 += tile)
    for (int64_t c = 0; c < L / 128; ++c) {
      const int64_t base = c * 128 * J + j0;
      const uint32_t nrec = records((L - c * 128) * J - j0);
      for (int w = 0; w < issuers; ++w)
        for (int k = 0; k < instr; ++k) {
          const int q = w + issuers * k;
          for (int lane = 0; lane < 64; ++lane) {
            const int r8 = lane >> 3, p8 = lane & 7;
            const int rr = 8 * (q & 15) + r8;
            const int piece = p8 ^ swz_slab(rr);
            const uint32_t voff = slab_lane(q, r8, piece, J);
            const int64_t row = c * 128 + rr;
            const int64_t col = j0 + 128 * (q >> 4) + 16 * piece;
            const bool in_range = voff < nrec;
            if (in_range) {
              const int64_t addr = base + voff;
              if (addr + 16 > L * J) fail("slab past end", L, J, row, col);
              if (col < J && addr != row * J + col) fail("slab address", row, col, addr, voff);
            } else if (col < J) {
              fail("slab valid column out of range", L, J, row, col);
            }
            if (row == L - 1 && col >= J && in_range) fail("slab last row", L, J, row, col);
          }
        }
    }
}

// Scale rows: one 64-lane load of 16 bytes per lane (four fp32 scales) from a resource of
// min(valid rows, tile) * 4 bytes.
static void check_scales(int64_t T, int tile) {
  for (int64_t t0 = 0; t0 < T; t0 += tile) {
    const int64_t valid = T - t0 < tile ? T - t0 : tile;
    const uint32_t nrec = records(valid * 4);
    for (int lane = 0; lane < 64; ++lane) {
      const uint32_t voff = 16 * lane;
      const bool in_range = voff < nrec;
      if (in_range != (4 * lane < valid)) fail("scale range", T, tile, lane, voff);
      if (in_range && t0 + 4 * lane + 4 > T) fail("scale past end", T, tile, lane, voff);
    }
  }
}

int main() {
  const int64_t dims[] = {128, 256, 384, 640, 1152, 2048, 2176};
  const int64_t reds[] = {128, 384, 2048};
  struct Plan {
    int tile, issuers;
  };
  // 256-row tiles: 8 waves issuing in alternating halves of 4; 192-row tiles: the same; 128-row
  // tiles: 4 waves (and the split-reduction kernel's two groups each issue as 4 waves).
  const Plan rows_plans[] = {{256, 4}, {192, 4}, {128, 4}};
  for (int64_t T : dims)
    for (int64_t L : reds)
      for (const Plan& p : rows_plans)
        if (T % 128 == 0 && (p.tile != 192 || T % 192 == 0)) check_rows(T, L, p.tile, p.issuers);
  const Plan slab_plans[] = {{256, 4}, {128, 4}};
  for (int64_t J : dims)
    for (int64_t L : reds)
      for (const Plan& p : slab_plans) check_slabs(L, J, p.tile, p.issuers);
  for (int64_t T : dims)
    for (int tile : {128, 192, 256}) check_scales(T, tile);
  if (failures) {
    std::printf("%d violations\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}

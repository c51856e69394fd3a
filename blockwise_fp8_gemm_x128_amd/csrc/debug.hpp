// Debug-mode input checks of libpuro (level set by puro_set_debug or the PURO_DEBUG environment
// variable). With the level at 0 every function here returns PURO_OK at once; otherwise it runs
// a check kernel on the caller's stream, waits for it, and returns PURO_ERR_INPUT when the data
// lies outside the entry points' contract.
#pragma once
#include <stdint.h>

#include "puro.h"

namespace puro {
namespace debug {

// Group shapes of a bf16 tensor's scale groups: 1x128 along each row, 128x1 along each column,
// 128x128 blocks.
enum Groups { kRowGroups = 1, kColGroups = 2, kBlockGroups = 4 };

bool on();

// bf16 input of a quantiser, rows x cols (multiples of 128): any NaN or infinity fails; with the
// amax/448 rule (pow2 false) so does any group of the given shapes whose largest magnitude is
// nonzero but below 2^-119.
puro_status check_bf16(const void* x, int64_t rows, int64_t cols, int groups, bool pow2,
                       void* stream);

// Operands of a GEMM: `codes` E4M3 bytes (an E4M3 NaN, 0x7F or 0xFF, fails) and `scales` fp32
// scales (anything but a positive finite value fails).
puro_status check_operand(const void* codes, int64_t ncodes, const float* scales,
                          int64_t nscales, void* stream);

}  // namespace debug
}  // namespace puro

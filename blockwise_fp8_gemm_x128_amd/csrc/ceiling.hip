// Measured ceilings of the MI355X matrix cores for the GEMMs' instruction (libpuro_probe.so).
//
// Not part of the GEMM path: a register-only microbenchmark that the measurement notes quote.
// Every wave loads 64 bytes of E4M3 codes per lane once (its A and B operands of one
// v_mfma_f32_16x16x128_f8f6f4), then runs `iters` rounds of kChains independent products on
// them, with nothing else in the loop but what the selected mode adds:
//   mode 0  the products accumulate in the matrix core (C = A*B + C): the instruction's own rate;
//   mode 1  each product starts from zero and is folded into an fp32 accumulator with 4 FMAs,
//           acc += s * P (the forward and data-gradient GEMMs' promotion: one scale per lane);
//   mode 2  as mode 1 with the scale formed per output column, 4 multiplies s_row * s_col[j]
//           and 4 FMAs (the weight-gradient GEMMs' promotion).
// The operand bytes are the caller's, so the rate can be measured on zero, random and
// quantised-data codes (the matrix cores draw more power, and the part clocks lower, on busy
// data). Each wave's lane 0 records the shader-clock cycles (s_memtime) and the constant-rate
// counter ticks (s_memrealtime) its loop took.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;

__device__ __forceinline__ v4f mfma(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int kMode>
__global__ void __launch_bounds__(1024)
    mfma_probe_kernel(const uint8_t* __restrict__ codes, int64_t nbytes, int64_t iters,
                      uint64_t* __restrict__ cycles, uint64_t* __restrict__ ticks,
                      float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  // nbytes is a multiple of 64, so the lane's 64 bytes lie inside the buffer
  const int64_t off = ((wave * 64 + lane) * 64) % nbytes;
  const v8i* src = reinterpret_cast<const v8i*>(codes + off);
  v8i a = src[0];
  v8i b = src[1];
  // per-chain start values and scales, hidden from the optimiser so that no two chains are
  // provably equal (they would be merged) and no scale product is provably loop-invariant
  v4f init[kChains];
  float s_row[kChains];  // one row scale per chain: each product has rows of its own
  v4f s_col = {1.0f, 1.0f + 0x1p-22f, 1.0f + 0x1p-21f, 1.0f + 0x1p-20f};
  asm volatile("" : "+v"(s_col));
#pragma unroll
  for (int k = 0; k < kChains; ++k) {
    init[k] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    s_row[k] = 1.0f + 0x1p-20f * (lane + 64 * k);
    asm volatile("" : "+v"(init[k]));
  }
  v4f acc[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) acc[k] = init[k];

  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t it = 0; it < iters; ++it) {
    // the operands (and scales) count as rewritten every round, so every product is issued
    asm volatile("" : "+v"(a), "+v"(b));
#pragma unroll
    for (int k = 0; k < kChains; ++k) asm volatile("" : "+v"(s_row[k]));
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
      if constexpr (kMode == 0) {
        acc[k] = mfma(a, b, acc[k]);
      } else {
        const v4f p = mfma(a, b, init[k]);
        if constexpr (kMode == 1) {
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[k][j] = __builtin_fmaf(s_row[k], p[j], acc[k][j]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[k][j] = __builtin_fmaf(s_row[k] * s_col[j], p[j], acc[k][j]);
        }
      }
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  sink[wave * 64 + lane] = s;
  if (lane == 0) {
    cycles[wave] = t1 - t0;
    ticks[wave] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// Runs the probe: `blocks` workgroups of `waves_per_block` waves (1-16), each wave `iters` rounds
// of 8 products (2*16*16*128 flop each) in the given mode (0, 1 or 2, above). codes: device
// buffer of code_bytes bytes (a multiple of 64, at least 4096, 64-byte aligned), read only.
// cycles, ticks: device arrays of blocks * waves_per_block uint64 (per wave: s_memtime and
// s_memrealtime deltas of its loop). sink: device array of 64 floats per wave (keeps the results
// live). The launch is
// asynchronous on `stream` (a hipStream_t, NULL for the default stream). Returns 0, 1 for an
// invalid argument, or 4 if the launch failed.
int puro_probe_mfma(const void* codes, int64_t code_bytes, int blocks, int waves_per_block,
                    int64_t iters, int mode, uint64_t* cycles, uint64_t* ticks, float* sink,
                    void* stream) {
  if (codes == nullptr || cycles == nullptr || ticks == nullptr || sink == nullptr) return 1;
  if (code_bytes < 4096 || code_bytes % 64 != 0) return 1;
  if ((reinterpret_cast<uintptr_t>(codes) & 63) != 0) return 1;
  if (blocks < 1 || blocks > (1 << 20) || waves_per_block < 1 || waves_per_block > 16) return 1;
  if (iters < 1 || mode < 0 || mode > 2) return 1;
  const dim3 grid(blocks), block(64 * waves_per_block);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* c = static_cast<const uint8_t*>(codes);
  if (mode == 0)
    hipLaunchKernelGGL(mfma_probe_kernel<0>, grid, block, 0, st, c, code_bytes, iters, cycles,
                       ticks, sink);
  else if (mode == 1)
    hipLaunchKernelGGL(mfma_probe_kernel<1>, grid, block, 0, st, c, code_bytes, iters, cycles,
                       ticks, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<2>, grid, block, 0, st, c, code_bytes, iters, cycles,
                       ticks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"

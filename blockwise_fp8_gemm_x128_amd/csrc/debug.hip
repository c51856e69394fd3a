// Debug-mode input checks (see debug.hpp and puro_set_debug in puro.h).
//
// The checks are plain scans, written for clarity rather than speed: they only run when the
// debug level is set. Their verdict goes to a per-device flag word in a file-scope device array
// whose address is looked up once per device; the host clears it with a one-thread kernel (no
// memset node), launches the scan, copies the word back and waits for the stream. A host mutex
// serialises checks, so threads that share a device do not read each other's verdicts.
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "common.hpp"
#include "debug.hpp"

namespace puro {
namespace {

__device__ __align__(16) uint32_t dbg_flags[4];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
uint32_t* g_flags[kMaxDevices] = {};
std::atomic<int> g_level{-1};  // -1: not read from the environment yet (lock-free reads: every
                              // quantiser and GEMM call asks)

// Flag bits
constexpr uint32_t kNonFinite = 1u;
constexpr uint32_t kTinyGroup = 2u;
constexpr uint32_t kNanCode = 4u;
constexpr uint32_t kBadScale = 8u;

// bf16 magnitude bits (sign cleared) as fp32 bits: finite values order like their bit patterns.
__device__ __forceinline__ uint32_t mag32(uint16_t v) {
  return static_cast<uint32_t>(v & 0x7fffu) << 16;
}
constexpr uint32_t kInfBits = 0x7f800000u;
constexpr uint32_t kTinyBits = 0x04000000u;  // 2^-119 as fp32 bits: (-119 + 127) << 23

__global__ void clear_kernel(uint32_t* flags) { flags[0] = 0u; }

// One 128-thread block per 128x128 tile: thread t scans row t of the tile (its 1x128 group) and
// column t (its 128x1 group); the block's maximum comes from the row maxima through LDS.
__global__ void __launch_bounds__(128)
    check_bf16_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int groups,
                      int tiny_check, uint32_t* __restrict__ flags) {
  const int64_t tiles_c = cols / 128;
  const int64_t r0 = (blockIdx.x / tiles_c) * 128, c0 = (blockIdx.x % tiles_c) * 128;
  const int t = threadIdx.x;
  uint32_t bad = 0, row_max = 0, col_max = 0;
  const uint16_t* row = x + (r0 + t) * cols + c0;
  for (int j = 0; j < 128; ++j) {
    const uint32_t m = mag32(row[j]);
    if (m >= kInfBits) bad |= kNonFinite;
    row_max = m > row_max ? m : row_max;
  }
  const uint16_t* col = x + r0 * cols + c0 + t;
  for (int i = 0; i < 128; ++i) {
    const uint32_t m = mag32(col[i * cols]);
    col_max = m > col_max ? m : col_max;
  }
  __shared__ uint32_t block_max;
  if (t == 0) block_max = 0;
  __syncthreads();
  atomicMax(&block_max, row_max);
  __syncthreads();
  auto tiny = [](uint32_t m) { return m != 0 && m < kTinyBits; };
  if (tiny_check) {
    if ((groups & debug::kRowGroups) && tiny(row_max)) bad |= kTinyGroup;
    if ((groups & debug::kColGroups) && tiny(col_max)) bad |= kTinyGroup;
    if ((groups & debug::kBlockGroups) && t == 0 && tiny(block_max)) bad |= kTinyGroup;
  }
  if (bad) atomicOr(flags, bad);
}

__global__ void check_codes_kernel(const uint8_t* __restrict__ q, int64_t n,
                                   uint32_t* __restrict__ flags) {
  uint32_t bad = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride)
    if ((q[i] & 0x7fu) == 0x7fu) bad |= kNanCode;
  if (bad) atomicOr(flags, bad);
}

__global__ void check_scales_kernel(const float* __restrict__ s, int64_t n,
                                    uint32_t* __restrict__ flags) {
  uint32_t bad = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride) {
    const float v = s[i];
    if (!(v > 0.0f && v <= 3.402823466e38f)) bad |= kBadScale;
  }
  if (bad) atomicOr(flags, bad);
}

// Device address of this device's flag word (looked up once per device).
puro_status flags_ptr(uint32_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PURO_ERR_LAUNCH;
  if (g_flags[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(dbg_flags)) != hipSuccess || p == nullptr)
      return PURO_ERR_LAUNCH;
    g_flags[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_flags[dev];
  return PURO_OK;
}

int level() {
  int l = g_level.load(std::memory_order_acquire);
  if (l < 0) {
    std::lock_guard<std::mutex> lock(g_mutex);
    l = g_level.load(std::memory_order_acquire);
    if (l < 0) {
      const char* e = getenv("PURO_DEBUG");
      l = (e != nullptr && atoi(e) > 0) ? atoi(e) : 0;
      g_level.store(l, std::memory_order_release);
    }
  }
  return l;
}

// Clear, run `scan`, read the verdict back. Called with g_mutex held.
template <class Scan>
puro_status run_check(void* stream, Scan scan) {
  uint32_t* flags = nullptr;
  PURO_TRY(flags_ptr(&flags));
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(1), 0, st, flags);
  if (hipGetLastError() != hipSuccess) return PURO_ERR_LAUNCH;
  scan(st, flags);
  if (hipGetLastError() != hipSuccess) return PURO_ERR_LAUNCH;
  uint32_t host = 0;
  if (hipMemcpyAsync(&host, flags, sizeof(host), hipMemcpyDeviceToHost, st) != hipSuccess)
    return PURO_ERR_LAUNCH;
  if (hipStreamSynchronize(st) != hipSuccess) return PURO_ERR_LAUNCH;
  return host == 0 ? PURO_OK : PURO_ERR_INPUT;
}

int scan_blocks(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return static_cast<int>(b < 4096 ? (b < 1 ? 1 : b) : 4096);
}

}  // namespace

namespace debug {

bool on() { return level() > 0; }

puro_status check_bf16(const void* x, int64_t rows, int64_t cols, int groups, bool pow2,
                       void* stream) {
  if (rows == 0 || cols == 0 || !on()) return PURO_OK;
  std::lock_guard<std::mutex> lock(g_mutex);
  const int64_t tiles = (rows / 128) * (cols / 128);
  if (tiles > INT32_MAX) return PURO_ERR_SHAPE;
  return run_check(stream, [&](hipStream_t st, uint32_t* flags) {
    hipLaunchKernelGGL(check_bf16_kernel, dim3(static_cast<uint32_t>(tiles)), dim3(128), 0, st,
                       static_cast<const uint16_t*>(x), rows, cols, groups, pow2 ? 0 : 1,
                       flags);
  });
}

puro_status check_operand(const void* codes, int64_t ncodes, const float* scales,
                          int64_t nscales, void* stream) {
  if (!on()) return PURO_OK;
  std::lock_guard<std::mutex> lock(g_mutex);
  return run_check(stream, [&](hipStream_t st, uint32_t* flags) {
    if (ncodes > 0)
      hipLaunchKernelGGL(check_codes_kernel, dim3(scan_blocks(ncodes)), dim3(256), 0, st,
                         static_cast<const uint8_t*>(codes), ncodes, flags);
    if (nscales > 0)
      hipLaunchKernelGGL(check_scales_kernel, dim3(scan_blocks(nscales)), dim3(256), 0, st,
                         scales, nscales, flags);
  });
}

}  // namespace debug
}  // namespace puro

extern "C" void puro_set_debug(int level) {
  puro::g_level.store(level > 0 ? level : 0, std::memory_order_release);
}

extern "C" int puro_debug_level(void) { return puro::level(); }

// Optimizer-step kernels for the fp32 master weights: the Frobenius-radius projection of the
// updated linear-layer matrices, and AdamW for the other parameters.
//
// Method: PuRo-2B news post (jj-blog-4lo.pages.dev), optimizer paragraph after the
// training-recipe paragraph — the matrices that are roughly scale-invariant get their update
// and are then scaled back to the Frobenius radius they had at initialisation, every step; the
// remaining parameters use AdamW. The masters stay fp32 (Paper walkthrough: Puro-2B, section
// "Lever 2: use blockwise FP8 from step zero"), and each updated matrix is also written as the
// bf16 copy the next step's 128x128 weight quantiser reads.
//
// All of it is HBM-bound streaming: 16 B per lane per access, grid-stride loops, and a
// deterministic two-level reduction (fp64 per lane and per block, then the block partials
// summed in one fixed order) whose grid depends on the element count only, so results are
// reproducible run to run and device to device.
#include <math.h>

#include <mutex>

#include "common.hpp"

namespace puro {
namespace {

// 16 bytes of an input read exactly once (the update direction, the gradient), loaded
// non-temporally so that it does not displace the masters, which the projected step reads twice
// (measured: the projected step 2 % faster).
__device__ __forceinline__ float4 load_once4f(const float4* p) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(t[0], t[1], t[2], t[3]);
}

constexpr int kOptThreads = 256;
constexpr int kOptMaxBlocks = PURO_OPT_MAX_BLOCKS;
// workspace layout: [kOptMaxBlocks] double partial sums
static_assert(sizeof(double) * kOptMaxBlocks <= PURO_OPT_WORKSPACE_BYTES, "workspace too small");

// Blocks of a reduction over n4 16-byte vectors: about four vectors per lane, at most
// kOptMaxBlocks.
inline int opt_blocks(int64_t n4) {
  const int64_t per_block = int64_t(kOptThreads) * 4;
  int64_t b = (n4 + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > kOptMaxBlocks) b = kOptMaxBlocks;
  return static_cast<int>(b);
}

__device__ __forceinline__ double block_sum(double x, double* sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  const int t = threadIdx.x;
  if ((t & 63) == 0) sh[t >> 6] = x;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

// Sum of squares, per block, of src (kUpdate false) or of v = src - lr*u, which is also
// written to dst (kUpdate true; dst may be src: the update is done in place).
template <bool kUpdate>
__global__ __launch_bounds__(kOptThreads) void sumsq_kernel(const float* src,
                                                            const float* __restrict__ u,
                                                            float* dst, int64_t n4, float lr,
                                                            double* __restrict__ partials) {
  __shared__ double sh[kOptThreads / 64];
  const float4* s4 = reinterpret_cast<const float4*>(src);
  const float4* u4 = reinterpret_cast<const float4*>(u);
  float4* d4 = reinterpret_cast<float4*>(dst);
  double acc = 0.0;
  for (int64_t i = int64_t(blockIdx.x) * kOptThreads + threadIdx.x; i < n4;
       i += int64_t(gridDim.x) * kOptThreads) {
    float4 a = s4[i];
    if constexpr (kUpdate) {
      const float4 b = load_once4f(u4 + i);
      a.x = fmaf(-lr, b.x, a.x);
      a.y = fmaf(-lr, b.y, a.y);
      a.z = fmaf(-lr, b.z, a.z);
      a.w = fmaf(-lr, b.w, a.w);
      d4[i] = a;
    }
    // each square of a binary32 is exact in binary64
    acc += (double(a.x) * a.x + double(a.y) * a.y) + (double(a.z) * a.z + double(a.w) * a.w);
  }
  const double s = block_sum(acc, sh);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

// Total of the block partials, summed in the same fixed order by whichever block asks (so every
// block of a launch gets the same value bit for bit).
__device__ __forceinline__ double total_of(const double* __restrict__ partials, int count,
                                          double* sh) {
  double acc = 0.0;
  for (int i = threadIdx.x; i < count; i += kOptThreads) acc += partials[i];
  return block_sum(acc, sh);
}

// One block: the norm.
__global__ __launch_bounds__(kOptThreads) void norm_kernel(const double* __restrict__ partials,
                                                           int count, float* __restrict__ norm) {
  __shared__ double sh[kOptThreads / 64];
  const double ss = total_of(partials, count, sh);
  if (threadIdx.x == 0) *norm = static_cast<float>(sqrt(ss));
}

__device__ __forceinline__ uint2 bf16x4(float4 a) {
  uint2 o;
  o.x = pack_bf16x2(a.x, a.y);
  o.y = pack_bf16x2(a.z, a.w);
  return o;
}

// w <- w * factor, and its bf16 copy. Every block first forms the factor radius / ||v|| itself
// from the partials (1 for a zero matrix, which has no direction to scale): 16 KB of cached
// reads per block instead of a dependent single-block launch.
__global__ __launch_bounds__(kOptThreads) void scale_kernel(float* __restrict__ w, int64_t n4,
                                                            const double* __restrict__ partials,
                                                            int count,
                                                            const float* __restrict__ radius,
                                                            uint16_t* __restrict__ wbf) {
  __shared__ double sh[kOptThreads / 64];
  const double ss = total_of(partials, count, sh);
  const float f = ss > 0.0 ? static_cast<float>(double(*radius) / sqrt(ss)) : 1.0f;
  float4* w4 = reinterpret_cast<float4*>(w);
  uint2* b4 = reinterpret_cast<uint2*>(wbf);
  for (int64_t i = int64_t(blockIdx.x) * kOptThreads + threadIdx.x; i < n4;
       i += int64_t(gridDim.x) * kOptThreads) {
    float4 a = w4[i];
    a.x *= f;
    a.y *= f;
    a.z *= f;
    a.w *= f;
    w4[i] = a;
    b4[i] = bf16x4(a);
  }
}

struct AdamWArgs {
  float lr, b1, omb1, b2, omb2, eps, decay, c1, c2;  // decay = 1 - lr*wd; c = 1 - beta^t
};

__device__ __forceinline__ void adamw_one(float& p, float g, float& m, float& v,
                                          const AdamWArgs& a) {
  m = fmaf(a.b1, m, a.omb1 * g);
  v = fmaf(a.b2, v, a.omb2 * (g * g));
  const float mh = m / a.c1;
  const float vh = v / a.c2;
  p = p * a.decay - a.lr * (mh / (sqrtf(vh) + a.eps));
}

template <bool kBf16>
__global__ __launch_bounds__(kOptThreads) void adamw_kernel(float* __restrict__ p,
                                                            const float* __restrict__ g,
                                                            float* __restrict__ m,
                                                            float* __restrict__ v, int64_t n4,
                                                            AdamWArgs a,
                                                            uint16_t* __restrict__ pbf) {
  float4* p4 = reinterpret_cast<float4*>(p);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  float4* m4 = reinterpret_cast<float4*>(m);
  float4* v4 = reinterpret_cast<float4*>(v);
  for (int64_t i = int64_t(blockIdx.x) * kOptThreads + threadIdx.x; i < n4;
       i += int64_t(gridDim.x) * kOptThreads) {
    float4 pp = p4[i], mm = m4[i], vv = v4[i];
    const float4 gg = load_once4f(g4 + i);
    adamw_one(pp.x, gg.x, mm.x, vv.x, a);
    adamw_one(pp.y, gg.y, mm.y, vv.y, a);
    adamw_one(pp.z, gg.z, mm.z, vv.z, a);
    adamw_one(pp.w, gg.w, mm.w, vv.w, a);
    p4[i] = pp;
    m4[i] = mm;
    v4[i] = vv;
    if constexpr (kBf16) reinterpret_cast<uint2*>(pbf)[i] = bf16x4(pp);
  }
}

// Elementwise kernels: enough blocks to fill the chip several times over, grid-stride beyond.
inline int stream_blocks(int64_t n4) {
  int64_t b = (n4 + kOptThreads - 1) / kOptThreads;
  if (b < 1) b = 1;
  if (b > 8192) b = 8192;
  return static_cast<int>(b);
}

inline bool numel_ok(int64_t n) { return n >= 0 && n % 4 == 0 && n <= (int64_t(1) << 40); }

// Scratch of the allocation-free projected step: the same partial sums the workspace argument
// holds, in a device array of the library's own. Its size does not depend on the element count
// (the reduction grid is capped at kOptMaxBlocks), so every valid call fits. Each device holds
// its own copy; host code uses the address hipGetSymbolAddress reports for the current device,
// never the array's name.
static __device__ __align__(256) uint8_t scratch[PURO_OPT_WORKSPACE_BYTES];
constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per device.
puro_status scratch_ptr(void** out) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PURO_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PURO_ERR_LAUNCH;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return PURO_OK;
}

}  // namespace
}  // namespace puro

using namespace puro;

extern "C" puro_status puro_frobenius_norm(const float* w, int64_t numel, float* norm,
                                           void* workspace, void* stream) {
  if (!numel_ok(numel)) return PURO_ERR_SHAPE;
  PURO_TRY(check_ptr(w, numel == 0));
  if (norm == nullptr || workspace == nullptr) return PURO_ERR_NULL;
  if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(norm) & 3u)) return PURO_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n4 = numel / 4;
  const int blocks = opt_blocks(n4);
  double* partials = static_cast<double*>(workspace);
  hipLaunchKernelGGL(sumsq_kernel<false>, dim3(blocks), dim3(kOptThreads), 0, s, w, nullptr,
                     nullptr, n4, 0.0f, partials);
  hipLaunchKernelGGL(norm_kernel, dim3(1), dim3(kOptThreads), 0, s, partials, blocks, norm);
  return launch_status();
}

extern "C" puro_status puro_hyperball_step(float* w, const float* u, int64_t numel, float lr,
                                           const float* radius, void* w_bf16, void* workspace,
                                           void* stream) {
  if (!numel_ok(numel)) return PURO_ERR_SHAPE;
  if (!isfinite(lr)) return PURO_ERR_ARG;
  const bool empty = numel == 0;
  PURO_TRY(check_ptr(w, empty));
  PURO_TRY(check_ptr(u, empty));
  PURO_TRY(check_ptr(w_bf16, empty));
  if (empty) return PURO_OK;
  if (radius == nullptr || workspace == nullptr) return PURO_ERR_NULL;
  if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(radius) & 3u)) return PURO_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n4 = numel / 4;
  const int blocks = opt_blocks(n4);
  double* partials = static_cast<double*>(workspace);
  hipLaunchKernelGGL(sumsq_kernel<true>, dim3(blocks), dim3(kOptThreads), 0, s, w, u, w, n4, lr,
                     partials);
  // the same grid as the reduction: each block re-sums the partials, so keep it small
  hipLaunchKernelGGL(scale_kernel, dim3(blocks), dim3(kOptThreads), 0, s, w, n4, partials, blocks,
                     radius, static_cast<uint16_t*>(w_bf16));
  return launch_status();
}

extern "C" puro_status puro_hyperball_step_noalloc(float* w, const float* u, int64_t numel,
                                                   float lr, const float* radius, void* w_bf16,
                                                   void* stream) {
  // the same validation as puro_hyperball_step, before anything touches the device
  if (!numel_ok(numel)) return PURO_ERR_SHAPE;
  if (!isfinite(lr)) return PURO_ERR_ARG;
  const bool empty = numel == 0;
  PURO_TRY(check_ptr(w, empty));
  PURO_TRY(check_ptr(u, empty));
  PURO_TRY(check_ptr(w_bf16, empty));
  if (empty) return PURO_OK;
  if (radius == nullptr) return PURO_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(radius) & 3u) return PURO_ERR_ALIGN;
  void* ws = nullptr;
  PURO_TRY(scratch_ptr(&ws));
  return puro_hyperball_step(w, u, numel, lr, radius, w_bf16, ws, stream);
}

extern "C" puro_status puro_adamw_step(float* p, const float* g, float* m, float* v,
                                       int64_t numel, const puro_adamw_params* hp, void* p_bf16,
                                       void* stream) {
  if (!numel_ok(numel)) return PURO_ERR_SHAPE;
  if (hp == nullptr) return PURO_ERR_NULL;
  if (hp->step < 1 || !(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) ||
      !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f) || !(hp->eps > 0.0f) || !isfinite(hp->lr) ||
      !isfinite(hp->weight_decay))
    return PURO_ERR_ARG;
  const bool empty = numel == 0;
  PURO_TRY(check_ptr(p, empty));
  PURO_TRY(check_ptr(g, empty));
  PURO_TRY(check_ptr(m, empty));
  PURO_TRY(check_ptr(v, empty));
  if (p_bf16 != nullptr && !aligned16(p_bf16)) return PURO_ERR_ALIGN;
  if (empty) return PURO_OK;
  AdamWArgs a;
  a.lr = hp->lr;
  a.b1 = hp->beta1;
  a.omb1 = 1.0f - hp->beta1;
  a.b2 = hp->beta2;
  a.omb2 = 1.0f - hp->beta2;
  a.eps = hp->eps;
  a.decay = static_cast<float>(1.0 - double(hp->lr) * double(hp->weight_decay));
  a.c1 = static_cast<float>(1.0 - pow(double(hp->beta1), double(hp->step)));
  a.c2 = static_cast<float>(1.0 - pow(double(hp->beta2), double(hp->step)));
  const int64_t n4 = numel / 4;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (p_bf16)
    hipLaunchKernelGGL(adamw_kernel<true>, dim3(stream_blocks(n4)), dim3(kOptThreads), 0, s, p,
                       g, m, v, n4, a, static_cast<uint16_t*>(p_bf16));
  else
    hipLaunchKernelGGL(adamw_kernel<false>, dim3(stream_blocks(n4)), dim3(kOptThreads), 0, s, p,
                       g, m, v, n4, a, nullptr);
  return launch_status();
}

// Measurement probes: kernels that each drive one hardware limit (the bf16
// matrix-core rate, HBM streaming copy, write and read), timed by the
// caller to obtain the peaks this GPU reaches. Contracts in include/gdn_probe.h.
#include <stdint.h>

#include "gdn_common.h"
#include "gdn_probe.h"

namespace {

using gdn::bf16x8;
using gdn::f32x4;

// Each wave: `iters` rounds of 8 independent MFMAs (8 accumulator chains, so the
// matrix pipe never waits on a result). The operands come from the lane index so
// that the compiler cannot fold the products; the accumulators' sum is stored.
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1.0f + 0.0078125f * ((lane + e) & 7));
    b[e] = static_cast<__bf16>(0.5f - 0.0078125f * ((lane * 3 + e) & 7));
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = gdn::zero4();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

// The streaming probes give each block one contiguous region (n / gridDim.x
// elements, rounded up; the last region ends at n) that its 256 lanes sweep in
// order, four 16-byte accesses in flight per lane: on MI355X this reaches
// 7.1 TB/s reading, 6.1 writing and 5.7 copying, where a grid-stride sweep
// (consecutive blocks on adjacent 4 KB pieces) reaches 6.2, 4.3 and 5.1.
__device__ __forceinline__ void block_region(int64_t n, int64_t& lo, int64_t& hi) {
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  lo = min(n, static_cast<int64_t>(blockIdx.x) * per);
  hi = min(n, lo + per);
}

__global__ __launch_bounds__(256) void copy_probe_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                         int64_t n) {
  int64_t lo, hi;
  block_region(n, lo, hi);
  int64_t i = lo + threadIdx.x;
  for (; i + 768 < hi; i += 1024) {
    const f32x4 a = __builtin_nontemporal_load(src + i);
    const f32x4 b = __builtin_nontemporal_load(src + i + 256);
    const f32x4 c = __builtin_nontemporal_load(src + i + 512);
    const f32x4 d = __builtin_nontemporal_load(src + i + 768);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + 256);
    __builtin_nontemporal_store(c, dst + i + 512);
    __builtin_nontemporal_store(d, dst + i + 768);
  }
  for (; i < hi; i += 256) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Streaming store of a constant (no reads).
__global__ __launch_bounds__(256) void write_probe_kernel(f32x4* __restrict__ dst, int64_t n) {
  int64_t lo, hi;
  block_region(n, lo, hi);
  const f32x4 x = f32x4{1.f, 2.f, 3.f, 4.f};
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256) __builtin_nontemporal_store(x, dst + i);
}

__global__ __launch_bounds__(256) void read_probe_kernel(const f32x4* __restrict__ src, float* __restrict__ sink,
                                                         int64_t n) {
  int64_t lo, hi;
  block_region(n, lo, hi);
  int64_t i = lo + threadIdx.x;
  f32x4 s0 = gdn::zero4(), s1 = gdn::zero4(), s2 = gdn::zero4(), s3 = gdn::zero4();
  for (; i + 768 < hi; i += 1024) {
    s0 += __builtin_nontemporal_load(src + i);
    s1 += __builtin_nontemporal_load(src + i + 256);
    s2 += __builtin_nontemporal_load(src + i + 512);
    s3 += __builtin_nontemporal_load(src + i + 768);
  }
  for (; i < hi; i += 256) s0 += __builtin_nontemporal_load(src + i);
  s0 += s1 + s2 + s3;
  float s = s0[0] + s0[1] + s0[2] + s0[3];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

constexpr int kStreamBlocks = 8192;  // 32 per CU: enough accesses in flight to saturate HBM

}  // namespace

extern "C" {

gdn_status gdn_probe_mfma_bf16(float* sink, int waves, int iters, void* stream) {
  if (!sink || !aligned16(sink) || waves <= 0 || waves % 4 || iters <= 0) return GDN_EINVAL;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(waves / 4), dim3(256), 0, static_cast<hipStream_t>(stream), sink,
                     iters);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || bytes <= 0 || bytes % 16) return GDN_EINVAL;
  hipLaunchKernelGGL(copy_probe_kernel, dim3(kStreamBlocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const gdn::f32x4*>(src), static_cast<gdn::f32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_probe_write(void* dst, int64_t bytes, void* stream) {
  if (!dst || !aligned16(dst) || bytes <= 0 || bytes % 16) return GDN_EINVAL;
  hipLaunchKernelGGL(write_probe_kernel, dim3(kStreamBlocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<gdn::f32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_probe_read(const void* src, float* sink, int64_t bytes, void* stream) {
  if (!src || !sink || !aligned16(src) || bytes <= 0 || bytes % 16) return GDN_EINVAL;
  hipLaunchKernelGGL(read_probe_kernel, dim3(kStreamBlocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const gdn::f32x4*>(src), sink, bytes / 16);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
}

}  // extern "C"

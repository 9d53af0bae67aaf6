// Device-side building blocks shared by the gfx950 kernels of the gated delta
// rule library: vector types, the 16x16x32 bf16 MFMA, fp32 -> bf16 hi/lo
// operand splitting, and the fragment index map all kernels agree on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 64;  // tokens per chunk (WarpDrive page, "Pipeline": C = 64)

// ---------------------------------------------------------------------------
// MFMA fragment conventions (v_mfma_f32_16x16x32_bf16, wave64).
//
// Lane l is split as g = l >> 4 (0..3) and c = l & 15.
//  * Accumulator D (16 x 16 fp32): lane (g, c) holds D[4g + r][c], r = 0..3.
//  * A operand (16 rows x 32 contraction): lane (g, c) holds row c at the
//    contraction indices kappa(g, e), e = 0..7.
//  * B operand (32 contraction x 16 cols): lane (g, c) holds column c at
//    kappa(g, e).
// kappa(g, e) = 4g + e for e < 4 and 16 + 4g + (e - 4) for e >= 4. Any bijection
// of the 32 contraction indices gives the same product as long as A and B use
// the same one; this one makes the two accumulator tiles covering rows
// [0, 16) and [16, 32) of a 32-row block exactly the B operand of that block
// ({tile0[0..3], tile1[0..3]} per lane), so a state held as accumulators feeds
// the next product with no data movement.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kappa(int g, int e) { return e < 4 ? 4 * g + e : 12 + 4 * g + e; }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }

// x ~= hi + lo with hi = RNE_bf16(x), lo = RNE_bf16(x - hi); |x - hi - lo| <= 2^-17 |x|.
__device__ __forceinline__ void split1(float x, __bf16& hi, __bf16& lo) {
  hi = to_bf16(x);
  lo = to_bf16(x - static_cast<float>(hi));
}

// Pack two accumulator tiles (rows [0,16) and [16,32) of a 32-row block) into the
// hi/lo B operand of that block.
__device__ __forceinline__ void split_tiles(const f32x4& t0, const f32x4& t1, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    __bf16 h, l;
    split1(t0[e], h, l);
    hi[e] = h;
    lo[e] = l;
    split1(t1[e], h, l);
    hi[4 + e] = h;
    lo[4 + e] = l;
  }
}

__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h, l;
    split1(x[e], h, l);
    hi[e] = h;
    lo[e] = l;
  }
}

// Products of split operands. A "part" count of 1 means the operand is exact
// in bf16 (lo == 0 and skipped); 2 means hi + lo. The lo x lo term is dropped.
template <int PA, int PB>
__device__ __forceinline__ f32x4 mma_split(bf16x8 ahi, bf16x8 alo, bf16x8 bhi, bf16x8 blo, f32x4 acc) {
  if constexpr (PB == 2) acc = mfma(ahi, blo, acc);
  if constexpr (PA == 2) acc = mfma(alo, bhi, acc);
  return mfma(ahi, bhi, acc);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 b) { return __builtin_bit_cast(u32x4, b); }

__device__ __forceinline__ bf16x8 zero_bf16x8() { return as_bf16x8(u32x4{0u, 0u, 0u, 0u}); }

// Load the 8 contraction-ordered elements kappa(g, 0..7) of a row whose
// 32-element block starts at p (element type bf16): two 8-byte loads.
__device__ __forceinline__ bf16x8 load_row_frag_bf16(const __bf16* p, int g) {
  u32x2 a = *reinterpret_cast<const u32x2*>(p + 4 * g);
  u32x2 b = *reinterpret_cast<const u32x2*>(p + 16 + 4 * g);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

// Same for a float32 row, split into hi/lo parts.
__device__ __forceinline__ void load_row_frag_f32(const float* p, int g, bf16x8& hi, bf16x8& lo) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * g);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 16 + 4 * g);
  float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  split8(x, hi, lo);
}

// Input element loading, for bf16 or float32 tensors.
template <typename T>
struct In;
template <>
struct In<__bf16> {
  static constexpr int kParts = 1;
  __device__ static __forceinline__ float ld(const __bf16* p) { return static_cast<float>(*p); }
  __device__ static __forceinline__ void row_frag(const __bf16* p, int g, bf16x8& hi, bf16x8& lo) {
    hi = load_row_frag_bf16(p, g);
    lo = zero_bf16x8();
  }
};
template <>
struct In<float> {
  static constexpr int kParts = 2;
  __device__ static __forceinline__ float ld(const float* p) { return *p; }
  __device__ static __forceinline__ void row_frag(const float* p, int g, bf16x8& hi, bf16x8& lo) {
    load_row_frag_f32(p, g, hi, lo);
  }
};

template <typename T>
__device__ __forceinline__ void store_out(T* p, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_out<__bf16>(__bf16* p, float x) { *p = to_bf16(x); }

// Wave-wide inclusive prefix sum over 64 lanes.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    float y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

}  // namespace gdn

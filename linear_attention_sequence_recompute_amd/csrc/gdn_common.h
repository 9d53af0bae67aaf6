// Device-side building blocks shared by the gfx950 kernels of the gated delta
// rule library: vector types, the MFMA instructions used, the fragment index map
// all kernels agree on, and the precision policies (how inputs and computed
// operands enter the matrix cores).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 64;  // tokens per chunk (WarpDrive page, "Pipeline": C = 64)

// ---------------------------------------------------------------------------
// MFMA fragment conventions (wave64, 16 x 16 output tiles).
//
// Lane l is split as g = l >> 4 (0..3) and c = l & 15.
//  * Accumulator D (16 x 16 fp32): lane (g, c) holds D[4g + r][c], r = 0..3.
//  * A operand (16 rows x 32 contraction): lane (g, c) holds row c at the
//    contraction indices kappa(g, e), e = 0..7.
//  * B operand (32 contraction x 16 cols): lane (g, c) holds column c at
//    kappa(g, e).
// kappa(g, e) = 4g + e for e < 4 and 16 + 4g + (e - 4) for e >= 4. Any bijection
// of the 32 contraction indices gives the same product as long as A and B use
// the same one; this one makes the two accumulator tiles covering rows [0, 16)
// and [16, 32) of a 32-row block exactly the B operand of that block
// ({tile0[0..3], tile1[0..3]} per lane), so a state held as accumulators feeds
// the next product with no data movement.
//
// With v_mfma_f32_16x16x32_bf16 a lane's 8 values go in one instruction. With
// v_mfma_f32_16x16x4f32 (lane (g, c) supplies contraction index g of row/column
// c) the same 32-deep product takes 8 instructions, the j-th feeding each lane's
// element j: together they cover every (g, e) pair once.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kappa(int g, int e) { return e < 4 ? 4 * g + e : 12 + 4 * g + e; }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 b) { return __builtin_bit_cast(u32x4, b); }
__device__ __forceinline__ bf16x8 zero_bf16x8() { return as_bf16x8(u32x4{0u, 0u, 0u, 0u}); }

// x ~= hi + lo with hi = RNE_bf16(x), lo = RNE_bf16(x - hi), |x - hi - lo| <= 2^-17 |x|,
// for a pair, packed: {hi(a), hi(b)} and {lo(a), lo(b)}. The residual x - hi is
// exact in fp32, so it is formed by a bf16 dot product of the packed hi pair
// with (-1, 0) or (0, -1) accumulated onto x, one instruction each.
// The two multiplier pairs are kept in registers (the empty asm hides their
// value): encoded as an inline constant, the pair (-1, 0) is not read back as
// that pair by v_dot2c_f32_bf16 on gfx950.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  uint32_t m0u = 0x0000bf80u, m1u = 0xbf800000u;  // {-1, 0}, {0, -1} (low half first)
  asm("" : "+v"(m0u));
  asm("" : "+v"(m1u));
  const bf16x2 m0 = __builtin_bit_cast(bf16x2, m0u);
  const bf16x2 m1 = __builtin_bit_cast(bf16x2, m1u);
  const float ra = __builtin_amdgcn_fdot2_f32_bf16(h, m0, a, false);
  const float rb = __builtin_amdgcn_fdot2_f32_bf16(h, m1, b, false);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{ra, rb}, bf16x2));
}

// ---------------------------------------------------------------------------
// Operand fragments: the 8 kappa-ordered values a lane contributes.
// ---------------------------------------------------------------------------
struct FragB {  // values exact in bf16 (bf16 inputs)
  bf16x8 x;
};
struct FragS {  // fp32 values carried as bf16 hi + lo (about 16 significant bits)
  bf16x8 hi, lo;
};
struct FragF {  // fp32 values (elements 0..3 in a, 4..7 in b)
  f32x4 a, b;
};

// Products accumulated in fp32, as a fixed sequence of MFMA instructions
// ("terms"): term(a, b, acc, t) issues the t-th, t < Terms<A, B>::n, so that
// code can interleave the terms of independent products. The lo x lo term of
// two split operands is dropped. Terms that use the hi half of a split operand
// come first: a split forms hi before lo, so the first MFMA can start earlier.
template <class A, class B>
struct Terms;
template <>
struct Terms<FragB, FragB> {
  static constexpr int n = 1;
};
template <>
struct Terms<FragB, FragS> {
  static constexpr int n = 2;
};
template <>
struct Terms<FragS, FragB> {
  static constexpr int n = 2;
};
template <>
struct Terms<FragS, FragS> {
  static constexpr int n = 3;
};
template <>
struct Terms<FragF, FragF> {
  static constexpr int n = 8;
};

__device__ __forceinline__ f32x4 term(const FragB& a, const FragB& b, f32x4 acc, int) { return mfma(a.x, b.x, acc); }
__device__ __forceinline__ f32x4 term(const FragB& a, const FragS& b, f32x4 acc, int t) {
  return mfma(a.x, t == 0 ? b.hi : b.lo, acc);
}
__device__ __forceinline__ f32x4 term(const FragS& a, const FragB& b, f32x4 acc, int t) {
  return mfma(t == 0 ? a.hi : a.lo, b.x, acc);
}
// (b is the operand split last in the scan: its hi half first)
__device__ __forceinline__ f32x4 term(const FragS& a, const FragS& b, f32x4 acc, int t) {
  return t == 0 ? mfma(a.hi, b.hi, acc) : t == 1 ? mfma(a.lo, b.hi, acc) : mfma(a.hi, b.lo, acc);
}
__device__ __forceinline__ f32x4 term(const FragF& a, const FragF& b, f32x4 acc, int t) {
  return t < 4 ? mfma_f32(a.a[t], b.a[t], acc) : mfma_f32(a.b[t - 4], b.b[t - 4], acc);
}

template <class A, class B>
__device__ __forceinline__ f32x4 mma(const A& a, const B& b, f32x4 acc) {
#pragma unroll
  for (int t = 0; t < Terms<A, B>::n; ++t) acc = term(a, b, acc, t);
  return acc;
}

// Scalar element loads of an input tensor.
__device__ __forceinline__ float ld_in(const __bf16* p) { return static_cast<float>(*p); }
__device__ __forceinline__ float ld_in(const float* p) { return *p; }

template <typename T>
__device__ __forceinline__ void store_out(T* p, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_out<__bf16>(__bf16* p, float x) { *p = to_bf16(x); }

// ---------------------------------------------------------------------------
// Precision policies. Prec<Tin> names the fragment types and conversions for
// inputs of type Tin:
//   In    fragments of q, k, v (exact: bf16 -> FragB, float -> FragF);
//   Cmp   fragments of computed operands (bf16 mode: FragS; float mode: FragF);
//   Stage element type of transposed input tiles staged in LDS;
//   Tile  an accumulator slice (4 rows of one column) in the form two of them
//         make a Cmp B operand (exchanged through LDS).
// A fragment is stored in memory as planes of 64 lanes x 16 bytes: FragB uses
// one plane, FragS (hi, lo) and FragF (a, b) two, so one lane's 16-byte load of
// a plane is fully coalesced across the wave.
// ---------------------------------------------------------------------------
template <typename Tin>
struct Prec;

template <>
struct Prec<__bf16> {
  using In = FragB;
  using Cmp = FragS;
  using Stage = __bf16;
  using Tile = u32x4;  // {hi bf16x4, lo bf16x4}
  static constexpr int kInPlanes = 1;

  __device__ static __forceinline__ In in_row(const __bf16* p, int g) {
    const u32x2 a = *reinterpret_cast<const u32x2*>(p + 4 * g);
    const u32x2 b = *reinterpret_cast<const u32x2*>(p + 16 + 4 * g);
    return In{as_bf16x8(u32x4{a[0], a[1], b[0], b[1]})};
  }
  __device__ static __forceinline__ In in_zero() { return In{zero_bf16x8()}; }
  __device__ static __forceinline__ In in_lds(const __bf16* row, int g) { return in_row(row, g); }
  __device__ static __forceinline__ Stage to_stage(float x) { return to_bf16(x); }
  __device__ static __forceinline__ void st_in(void* base, int lane, const In& f) {
    reinterpret_cast<u32x4*>(base)[lane] = as_u32x4(f.x);
  }
  __device__ static __forceinline__ In ld_in_frag(const void* base, int lane) {
    return In{as_bf16x8(reinterpret_cast<const u32x4*>(base)[lane])};
  }

  __device__ static __forceinline__ Cmp cmp8(const float (&x)[8]) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split2(x[2 * e], x[2 * e + 1], h[e], l[e]);
    return Cmp{as_bf16x8(u32x4{h[0], h[1], h[2], h[3]}), as_bf16x8(u32x4{l[0], l[1], l[2], l[3]})};
  }
  __device__ static __forceinline__ Cmp cmp_tiles(const f32x4& t0, const f32x4& t1) {
    const float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
    return cmp8(x);
  }
  __device__ static __forceinline__ void st_cmp(void* base, int lane, const Cmp& f) {
    reinterpret_cast<u32x4*>(base)[lane] = as_u32x4(f.hi);
    reinterpret_cast<u32x4*>(base)[64 + lane] = as_u32x4(f.lo);
  }
  __device__ static __forceinline__ Cmp ld_cmp(const void* base, int lane) {
    return Cmp{as_bf16x8(reinterpret_cast<const u32x4*>(base)[lane]),
               as_bf16x8(reinterpret_cast<const u32x4*>(base)[64 + lane])};
  }
  __device__ static __forceinline__ Tile tile(const f32x4& t) {
    uint32_t h0, h1, l0, l1;
    split2(t[0], t[1], h0, l0);
    split2(t[2], t[3], h1, l1);
    return Tile{h0, h1, l0, l1};
  }
  __device__ static __forceinline__ Cmp cmp_from(const Tile& t0, const Tile& t1) {
    return Cmp{as_bf16x8(u32x4{t0[0], t0[1], t1[0], t1[1]}), as_bf16x8(u32x4{t0[2], t0[3], t1[2], t1[3]})};
  }
  // A-operand fragment of the transpose of a row-major LDS tile: rows of the
  // fragment are tile columns [col0, col0 + 16), its contraction runs over tile
  // rows [row0, row0 + 32). Uses ds_read_b64_tr_b16: within a group of 16 lanes,
  // output lane j receives element j & 3 of the 4 loaded by lane 4e + (j >> 2) as
  // its element e, so lane l' of group g loads 4 consecutive columns of tile row
  // row0 + 4g + (l' >> 2) (+ 16 for the second half of the fragment).
  __device__ static __forceinline__ In in_lds_tr(const Stage* tile, int stride, int row0, int col0, int lane) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const int g = lane >> 4, l = lane & 15;
    const Stage* p0 = tile + (row0 + 4 * g + (l >> 2)) * stride + col0 + 4 * (l & 3);
    const Stage* p1 = p0 + 16 * stride;
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
    const u32x2 au = __builtin_bit_cast(u32x2, a), bu = __builtin_bit_cast(u32x2, b);
    return In{as_bf16x8(u32x4{au[0], au[1], bu[0], bu[1]})};
  }
  // Writes accumulator tile t (4 rows of one column per lane) as half `half` of
  // the stored B-operand fragment at `base` (planes as in st_cmp): rows [0, 16) of
  // a 32-row block are half 0, rows [16, 32) half 1.
  __device__ static __forceinline__ void st_tile(void* base, int lane, int half, const f32x4& t) {
    const Tile v = tile(t);
    char* b = static_cast<char*>(base) + lane * 16 + half * 8;
    *reinterpret_cast<u32x2*>(b) = u32x2{v[0], v[1]};
    *reinterpret_cast<u32x2*>(b + 1024) = u32x2{v[2], v[3]};
  }
};

template <>
struct Prec<float> {
  using In = FragF;
  using Cmp = FragF;
  using Stage = float;
  using Tile = f32x4;
  static constexpr int kInPlanes = 2;

  __device__ static __forceinline__ In in_row(const float* p, int g) {
    return In{*reinterpret_cast<const f32x4*>(p + 4 * g), *reinterpret_cast<const f32x4*>(p + 16 + 4 * g)};
  }
  __device__ static __forceinline__ In in_zero() { return In{zero4(), zero4()}; }
  __device__ static __forceinline__ In in_lds(const float* row, int g) { return in_row(row, g); }
  __device__ static __forceinline__ Stage to_stage(float x) { return x; }
  __device__ static __forceinline__ void st_in(void* base, int lane, const In& f) { st_cmp(base, lane, f); }
  __device__ static __forceinline__ In ld_in_frag(const void* base, int lane) { return ld_cmp(base, lane); }

  __device__ static __forceinline__ Cmp cmp8(const float (&x)[8]) {
    return Cmp{f32x4{x[0], x[1], x[2], x[3]}, f32x4{x[4], x[5], x[6], x[7]}};
  }
  __device__ static __forceinline__ Cmp cmp_tiles(const f32x4& t0, const f32x4& t1) { return Cmp{t0, t1}; }
  __device__ static __forceinline__ void st_cmp(void* base, int lane, const Cmp& f) {
    reinterpret_cast<f32x4*>(base)[lane] = f.a;
    reinterpret_cast<f32x4*>(base)[64 + lane] = f.b;
  }
  __device__ static __forceinline__ Cmp ld_cmp(const void* base, int lane) {
    return Cmp{reinterpret_cast<const f32x4*>(base)[lane], reinterpret_cast<const f32x4*>(base)[64 + lane]};
  }
  __device__ static __forceinline__ Tile tile(const f32x4& t) { return t; }
  __device__ static __forceinline__ Cmp cmp_from(const Tile& t0, const Tile& t1) { return Cmp{t0, t1}; }
  __device__ static __forceinline__ In in_lds_tr(const Stage* tile, int stride, int row0, int col0, int lane) {
    const int g = lane >> 4, c = lane & 15;
    In f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f.a[e] = tile[(row0 + 4 * g + e) * stride + col0 + c];
      f.b[e] = tile[(row0 + 16 + 4 * g + e) * stride + col0 + c];
    }
    return f;
  }
  __device__ static __forceinline__ void st_tile(void* base, int lane, int half, const f32x4& t) {
    reinterpret_cast<f32x4*>(base)[half * 64 + lane] = t;
  }
};

// ---------------------------------------------------------------------------
// Buffer addressing: a resource descriptor (base address and size in bytes, in
// scalar registers) plus a 32-bit per-lane offset and a uniform offset. Loads
// past the size return zeros and stores past it are dropped, so a descriptor
// that ends at a chunk's last row masks the rows beyond it without branches.
// ---------------------------------------------------------------------------
struct Buf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ Buf(const void* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000)) {}
  __device__ __forceinline__ u32x4 load16(uint32_t voff, uint32_t soff) const {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  }
  // 16 bytes per lane straight into LDS: lane i's bytes land at lds_block + 16 i
  // (lds_block must be the same for all lanes).
  __device__ __forceinline__ void to_lds16(void* lds_block, uint32_t voff, uint32_t soff) const {
    const uint32_t l = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_block));  // LDS offset
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(static_cast<uintptr_t>(l)), 16,
                                             voff, soff, 0, 0);
  }
  // 4 bytes per lane straight into LDS (lane i's at lds_block + 4 i).
  __device__ __forceinline__ void to_lds4(void* lds_block, uint32_t voff, uint32_t soff) const {
    const uint32_t l = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_block));  // LDS offset
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(static_cast<uintptr_t>(l)), 4,
                                             voff, soff, 0, 0);
  }
  // 4 bytes per lane (0 for lanes with voff >= the descriptor size).
  __device__ __forceinline__ uint32_t load4(uint32_t voff) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
  }
  // 2 bytes per lane (0 past the descriptor size).
  __device__ __forceinline__ uint16_t load2(uint32_t voff, uint32_t soff) const {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  }
  __device__ __forceinline__ void store(float x, uint32_t voff, uint32_t soff) const {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, voff, soff, 0);
  }
  __device__ __forceinline__ void store(__bf16 x, uint32_t voff, uint32_t soff) const {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r, voff, soff, 0);
  }
};

// Wave-wide inclusive prefix sum over 64 lanes.
// x of lane (lane ^ 1) or (lane ^ 2) within each group of four lanes, by a DPP
// quad permutation (no LDS round trip, unlike a general shuffle).
__device__ __forceinline__ float quad_xor1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
}

// Workgroup w of a grid of npages x NP workgroups -> (page, part): the decode
// kernels' state pages (one per request and head), NP workgroups each. The 8
// XCDs take workgroups round-robin (w mod 8); where the page count allows, XCD x
// is given a contiguous eighth of the pages, in order and each page's NP parts
// back to back, so that every XCD streams whole pages through its own L2 (on
// MI355X the decode step moves 6.1 TB/s this way, 5.8 with consecutive
// workgroups spread over the XCDs). A bijection onto [0, npages) x [0, NP).
template <int NP>
__device__ __forceinline__ void xcd_page_part(int w, int npages, int& page, int& part) {
  if (npages % 8 == 0) {
    const int r = w >> 3;
    part = r % NP;
    page = (w & 7) * (npages / 8) + r / NP;
  } else {
    page = w / NP;
    part = w % NP;
  }
}

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

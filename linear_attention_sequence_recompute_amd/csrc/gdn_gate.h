// The per-key-channel decay ("gate") of the KDA decode layer (the vLLM KdaSplit
// page, method gate_warp), shared by the gate stage's own kernel and the decode
// layer that computes its decays in place: for one token and one (head, key
// channel) row of F_B,
//   raw = f_a . F_B[row]   (float32, R = 128 terms, in the order the gate mode fixes)
//   log_decay = lower_bound * sigmoid(exp(a_log[h]) * (bf16(raw) + dt_bias[row]))
// The projection is kept in IEEE float32 (the page says so): plain fused
// multiply-adds and adds in a fixed order, so that the bf16 rounding of raw is
// reproducible. Modes: 0, one chain over the 128 columns; 1, four chains of 32
// columns summed as 0 + (((c0 + c1) + c2) + c3); 2, sixteen partials of 8
// columns summed in a butterfly (p[i] += p[i + 2^s], s = 3, 2, 1, 0). The page
// runs modes 0 and 1 as chains of 16-column MMA blocks; the order inside a block
// is read here as column order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kGateRank = 128;

// raw for mode MODE; x(c) and w(c) give column c of the activations and of the
// weight row as floats. A scheduling barrier after every 32 columns keeps one
// chunk of unpacked operands live at a time.
template <int MODE, class X, class W>
__device__ __forceinline__ float gate_raw(X x, W w) {
  constexpr int R = kGateRank;
  auto chunk_end = [](int c4) {
    if (c4 % 8 == 7) __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (MODE == 0) {
    float acc = 0.f;
#pragma unroll
    for (int c4 = 0; c4 < R / 4; ++c4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(x(4 * c4 + e), w(4 * c4 + e), acc);
      // the chain pinned at each chunk end, so that a chunk's FMAs stay ahead of
      // the next chunk's activation loads (issued all at once, the loads held the
      // whole row in scalar registers, which then spilled into vector lanes)
      if (c4 % 8 == 7) asm volatile("" : "+v"(acc));
      chunk_end(c4);
    }
    return acc;
  } else if constexpr (MODE == 1) {
    float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c4 = 0; c4 < R / 4; ++c4) {
      const int j = c4 / 8;  // 32 columns per chain
#pragma unroll
      for (int e = 0; e < 4; ++e) p[j] = fmaf(x(4 * c4 + e), w(4 * c4 + e), p[j]);
      chunk_end(c4);
    }
    return 0.f + (((p[0] + p[1]) + p[2]) + p[3]);
  } else {
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = 0.f;
#pragma unroll
    for (int c4 = 0; c4 < R / 4; ++c4) {
      const int i = c4 / 2;  // 8 columns per partial
#pragma unroll
      for (int e = 0; e < 4; ++e) p[i] = fmaf(x(4 * c4 + e), w(4 * c4 + e), p[i]);
      chunk_end(c4);
    }
#pragma unroll
    for (int sh = 3; sh >= 0; --sh)
#pragma unroll
      for (int i = 0; i < (1 << sh); ++i) p[i] = p[i] + p[i | (1 << sh)];
    return p[0];
  }
}

// The log-decay from the bf16-rounded projection rg (ea = exp(a_log[h])).
__device__ __forceinline__ float gate_log_decay(__bf16 rg, float ea, float dt, float lower_bound) {
  const float pre = ea * (static_cast<float>(rg) + dt);
  const float gate = 1.f / (1.f + expf(-pre));
  return lower_bound * gate;
}

// Column c of a bf16 row stored as 32-bit pairs (low half first), as float.
__device__ __forceinline__ float bf16_pair_col(const uint32_t* row, int c) {
  const uint32_t u = row[c >> 1];
  return __uint_as_float((c & 1) ? (u & 0xffff0000u) : (u << 16));
}

}  // namespace gdn

// The per-key-channel decay ("gate") stage of the KDA decode layer (the vLLM
// KdaSplit page, method gate_warp): for token t, head h and key channel f,
//   raw = f_a[t, :] . F_B[h K + f, :]   (float32, R = 128 terms, in the order the
//                                         gate mode fixes)
//   log_decay = lower_bound * sigmoid(exp(a_log[h]) * (bf16(raw) + dt_bias[h K + f]))
// The projection is kept in IEEE float32 (the page says so): plain fused
// multiply-adds and adds in a fixed order, so that the bf16 rounding of raw is
// reproducible. Modes: 0, one chain over the 128 columns; 1, four chains of 32
// columns summed as 0 + (((c0 + c1) + c2) + c3); 2, sixteen partials of 8
// columns summed in a butterfly (p[i] += p[i + 2^s], s = 3, 2, 1, 0). The page
// runs modes 0 and 1 as chains of 16-column MMA blocks; the order inside a block
// is read here as column order.
//
// One workgroup per (block of kGateTok tokens, head), one thread per key
// channel: the thread's F_B row lives in registers as float32; each token's
// activations are read once per wave into scalar registers.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kGateRank = 128;
constexpr int kGateTok = 8;  // tokens per workgroup

__device__ __forceinline__ void unpack8(const u32x4& u, float* dst) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dst[2 * i] = __uint_as_float(u[i] << 16);
    dst[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}

template <int K, int MODE>
__global__ __launch_bounds__(K) void kda_gate_kernel(const __bf16* __restrict__ f_a, const __bf16* __restrict__ f_b,
                                                     const float* __restrict__ a_log,
                                                     const float* __restrict__ dt_bias, float lower_bound,
                                                     float* __restrict__ g, __bf16* __restrict__ raw_out, int N,
                                                     int H) {
  constexpr int R = kGateRank;
  const int f = threadIdx.x, h = blockIdx.y;
  const int t0 = blockIdx.x * kGateTok;
  const int nt = min(kGateTok, N - t0);
  float w[R];
  const __bf16* wr = f_b + (static_cast<int64_t>(h) * K + f) * R;
#pragma unroll
  for (int c8 = 0; c8 < R / 8; ++c8) unpack8(*reinterpret_cast<const u32x4*>(wr + 8 * c8), &w[8 * c8]);
  const float ea = expf(a_log[h]);
  const float dt = dt_bias[h * K + f];

  // one token at a time (a wave issues dependent VALU operations back to back);
  // the token's activations are the same for every lane: uniform loads, which
  // the compiler places in scalar registers
  for (int t = 0; t < nt; ++t) {
    const uint32_t* xr = reinterpret_cast<const uint32_t*>(f_a) + static_cast<int64_t>(t0 + t) * (R / 2);
    // column c of the token as float32 (bf16 pairs, low half first)
    auto x = [&](int c) {
      const uint32_t u = xr[c >> 1];
      return __uint_as_float((c & 1) ? (u & 0xffff0000u) : (u << 16));
    };
    // keeps one 32-column chunk of unpacked activations live at a time
    auto chunk_end = [](int c4) {
      if (c4 % 8 == 7) __builtin_amdgcn_sched_barrier(0);
    };
    float raw;
    if constexpr (MODE == 0) {
      float acc = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < R / 4; ++c4) {
        acc = fmaf(x(4 * c4), w[4 * c4], acc);
        acc = fmaf(x(4 * c4 + 1), w[4 * c4 + 1], acc);
        acc = fmaf(x(4 * c4 + 2), w[4 * c4 + 2], acc);
        acc = fmaf(x(4 * c4 + 3), w[4 * c4 + 3], acc);
        chunk_end(c4);
      }
      raw = acc;
    } else if constexpr (MODE == 1) {
      float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c4 = 0; c4 < R / 4; ++c4) {
        const int j = c4 / 8;  // 32 columns per chain
        p[j] = fmaf(x(4 * c4), w[4 * c4], p[j]);
        p[j] = fmaf(x(4 * c4 + 1), w[4 * c4 + 1], p[j]);
        p[j] = fmaf(x(4 * c4 + 2), w[4 * c4 + 2], p[j]);
        p[j] = fmaf(x(4 * c4 + 3), w[4 * c4 + 3], p[j]);
        chunk_end(c4);
      }
      raw = 0.f + (((p[0] + p[1]) + p[2]) + p[3]);
    } else {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < R / 4; ++c4) {
        const int i = c4 / 2;  // 8 columns per partial
        p[i] = fmaf(x(4 * c4), w[4 * c4], p[i]);
        p[i] = fmaf(x(4 * c4 + 1), w[4 * c4 + 1], p[i]);
        p[i] = fmaf(x(4 * c4 + 2), w[4 * c4 + 2], p[i]);
        p[i] = fmaf(x(4 * c4 + 3), w[4 * c4 + 3], p[i]);
        chunk_end(c4);
      }
#pragma unroll
      for (int sh = 3; sh >= 0; --sh)
#pragma unroll
        for (int i = 0; i < (1 << sh); ++i) p[i] = p[i] + p[i | (1 << sh)];
      raw = p[0];
    }
    const __bf16 rg = static_cast<__bf16>(raw);  // round to nearest even
    const float pre = ea * (static_cast<float>(rg) + dt);
    const float gate = 1.f / (1.f + expf(-pre));
    const int64_t o = (static_cast<int64_t>(t0 + t) * H + h) * K + f;
    g[o] = lower_bound * gate;
    if (raw_out) raw_out[o] = rg;
  }
}

template <int K>
static void launch_gate_k(const GateArgs& a) {
  const dim3 grid(static_cast<unsigned>((a.N + kGateTok - 1) / kGateTok), static_cast<unsigned>(a.H));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(K), 0, a.stream, static_cast<const __bf16*>(a.f_a),
                       static_cast<const __bf16*>(a.f_b), a.a_log, a.dt_bias, a.lower_bound, a.g,
                       static_cast<__bf16*>(a.raw_out), a.N, a.H);
  };
  if (a.mode == 0)
    go(kda_gate_kernel<K, 0>);
  else if (a.mode == 1)
    go(kda_gate_kernel<K, 1>);
  else
    go(kda_gate_kernel<K, 2>);
}

hipError_t launch_kda_gate(const GateArgs& a) {
  if (a.K == 128)
    launch_gate_k<128>(a);
  else
    launch_gate_k<64>(a);
  return hipGetLastError();
}

}  // namespace gdn

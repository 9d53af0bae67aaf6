// Front and back operations of the decode layer around the recurrent step (the
// vLLM KdaSplit page, kernel body): before it, a causal depthwise convolution of 4
// taps over the conv-state pool (the slot's last three inputs, then the token's),
// SiLU, the per-head L2 norm of q and k (1e-6 inside the square root) and
// beta = sigmoid(raw beta); after it, the gated RMSNorm of each head's output,
// o * rsqrt(mean(o^2) + eps) * w * sigmoid(gate). That page fuses these steps into
// its decode kernel; here they are two small kernels beside the decode step.
//
// D / 2 lanes per head, two adjacent channels per lane (D = 64 or 128): each lane
// convolves its channels of the three sections (q, k, v) with dword and float2
// accesses, and the head's sums of squares reduce by wave shuffles.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

// Lanes of one (request, head) row: two channels each, so a head of D channels
// takes D / 2 consecutive lanes and its sums reduce by shuffles alone.
template <int D>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int m = D / 4; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack(uint32_t lo, uint32_t hi) { return (lo & 0xffffu) | (hi << 16); }

struct alignas(4) Dw3 {
  uint32_t w[3];
};

constexpr int kLayerThreads = 256;
constexpr int kPrologueReqs = 4;  // requests per lane group: the head's weights are loaded once for them

// A group of D / 2 lanes takes one head for kPrologueReqs consecutive requests,
// one lane per two adjacent channels c, c + 1. The head's conv weights and bias
// stay in registers across the requests. The two channels' conv state is 6
// consecutive bf16 (c: oldest..newest, then c + 1), read and written as three
// dwords; inputs and outputs move as dword or float2 pairs.
template <int D, bool BIAS>
__global__ __launch_bounds__(kLayerThreads) void decode_prologue_kernel(
    const __bf16* __restrict__ x, const float* __restrict__ conv_w, const float* __restrict__ conv_bias,
    __bf16* __restrict__ conv_state, int64_t pool_slots, const int32_t* __restrict__ slots,
    const float* __restrict__ beta_raw, float* __restrict__ q, float* __restrict__ k, float* __restrict__ v,
    float* __restrict__ beta, int N, int H, int64_t groups) {
  constexpr int LPH = D / 2;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kLayerThreads + threadIdx.x;
  const int64_t grp = gid / LPH;  // (request block, head)
  if (grp >= groups) return;      // whole groups leave together: groups are LPH-lane aligned
  const int c = 2 * static_cast<int>(gid % LPH);
  const int h = static_cast<int>(grp % H);
  const int64_t b0 = (grp / H) * kPrologueReqs;
  const int64_t dim = static_cast<int64_t>(H) * D, C = 3 * dim;
  // All loads of the group's requests first (their conv states share one pointer
  // with the stores below, so they would not be moved above them); the slots
  // lead, as the conv-state addresses wait on them.
  int slot[kPrologueReqs];
  bool live[kPrologueReqs];
  Dw3 st[kPrologueReqs][3];
  uint32_t xw[kPrologueReqs][3];
#pragma unroll
  for (int r = 0; r < kPrologueReqs; ++r) {
    const int64_t b = b0 + r;
    slot[r] = b < N ? slots[b] : 0;
  }
  float2 w[3][4], bias[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int64_t ch = s * dim + static_cast<int64_t>(h) * D + c;
    const float* wc = conv_w + (s * 4) * dim + static_cast<int64_t>(h) * D + c;  // weights [3][4][dim]
#pragma unroll
    for (int i = 0; i < 4; ++i) w[s][i] = *reinterpret_cast<const float2*>(wc + i * dim);
    bias[s] = BIAS ? *reinterpret_cast<const float2*>(conv_bias + ch) : make_float2(0.f, 0.f);
  }
#pragma unroll
  for (int r = 0; r < kPrologueReqs; ++r) live[r] = slot[r] > 0 && slot[r] < pool_slots;
#pragma unroll
  for (int r = 0; r < kPrologueReqs; ++r) {
    if (!live[r]) continue;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int64_t ch = s * dim + static_cast<int64_t>(h) * D + c;
      st[r][s] = *reinterpret_cast<const Dw3*>(conv_state + (static_cast<int64_t>(slot[r]) * C + ch) * 3);
      xw[r][s] = *reinterpret_cast<const uint32_t*>(x + (b0 + r) * C + ch);
    }
  }
#pragma unroll
  for (int r = 0; r < kPrologueReqs; ++r) {
    const int64_t b = b0 + r;
    if (b >= N) break;
    const int64_t row = b * H + h;
    const int64_t out = row * D + c;
    if (!live[r]) {  // padding: zero outputs, conv state untouched
      const float2 z = make_float2(0.f, 0.f);
      *reinterpret_cast<float2*>(q + out) = z;
      *reinterpret_cast<float2*>(k + out) = z;
      *reinterpret_cast<float2*>(v + out) = z;
      if (c == 0) beta[row] = 0.f;
      continue;
    }
    float2 y[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int64_t ch = s * dim + static_cast<int64_t>(h) * D + c;
      const Dw3& t = st[r][s];
      const uint32_t xs = xw[r][s];
      float2 acc = bias[s];
      // channel c: state (lo0, hi0, lo1); channel c + 1: (hi1, lo2, hi2)
      acc.x = fmaf(w[s][0].x, bf_lo(t.w[0]), acc.x);
      acc.x = fmaf(w[s][1].x, bf_hi(t.w[0]), acc.x);
      acc.x = fmaf(w[s][2].x, bf_lo(t.w[1]), acc.x);
      acc.x = fmaf(w[s][3].x, bf_lo(xs), acc.x);
      acc.y = fmaf(w[s][0].y, bf_hi(t.w[1]), acc.y);
      acc.y = fmaf(w[s][1].y, bf_lo(t.w[2]), acc.y);
      acc.y = fmaf(w[s][2].y, bf_hi(t.w[2]), acc.y);
      acc.y = fmaf(w[s][3].y, bf_hi(xs), acc.y);
      y[s].x = acc.x / (1.f + expf(-acc.x));  // SiLU
      y[s].y = acc.y / (1.f + expf(-acc.y));
      Dw3 ns;
      ns.w[0] = pack(t.w[0] >> 16, t.w[1]);   // c: t1, t2
      ns.w[1] = pack(xs, t.w[2]);              // c: x; c + 1: t1
      ns.w[2] = pack(t.w[2] >> 16, xs >> 16);  // c + 1: t2, x
      *reinterpret_cast<Dw3*>(conv_state + (static_cast<int64_t>(slot[r]) * C + ch) * 3) = ns;
    }
    const float nq = row_sum<D>(y[0].x * y[0].x + y[0].y * y[0].y);
    const float nk = row_sum<D>(y[1].x * y[1].x + y[1].y * y[1].y);
    const float rq = rsqrtf(nq + 1e-6f), rk = rsqrtf(nk + 1e-6f);
    *reinterpret_cast<float2*>(q + out) = make_float2(y[0].x * rq, y[0].y * rq);
    *reinterpret_cast<float2*>(k + out) = make_float2(y[1].x * rk, y[1].y * rk);
    *reinterpret_cast<float2*>(v + out) = y[2];
    if (c == 0) beta[row] = 1.f / (1.f + expf(-beta_raw[row]));
  }
}

// The front for T tokens per request (speculative verify, the KdaSplit class
// docstring and the kernel body's tokens branch): the conv page of slot[b, 0]
// holds T + 2 inputs per channel; token t convolves (page columns a - 1, a, a + 1,
// then x_0 .. x_{T-1}) at positions t .. t + 3 (a = accepted[b]), and the page
// becomes (column a, column a + 1, x_0 .. x_{T-1}). A group of D / 2 lanes takes
// one (request, head), two adjacent channels per lane, and runs the T tokens in
// a sliding window held in registers; every tap is read before the page is
// rewritten (each lane reads and writes only its own channels).
template <int D, bool BIAS>
__global__ __launch_bounds__(kLayerThreads) void decode_prologue_verify_kernel(
    const __bf16* __restrict__ x, const float* __restrict__ conv_w, const float* __restrict__ conv_bias,
    __bf16* __restrict__ conv_state, int64_t pool_slots, const int32_t* __restrict__ slots, int cols,
    const int32_t* __restrict__ accepted, const float* __restrict__ beta_raw, float* __restrict__ q,
    float* __restrict__ k, float* __restrict__ v, float* __restrict__ beta, int N, int T, int H) {
  constexpr int LPH = D / 2;
  constexpr int kMaxT = 8;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kLayerThreads + threadIdx.x;
  const int64_t grp = gid / LPH;  // (request, head)
  if (grp >= static_cast<int64_t>(N) * H) return;  // whole groups leave together
  const int c = 2 * static_cast<int>(gid % LPH);
  const int h = static_cast<int>(grp % H);
  const int64_t b = grp / H;
  const int64_t dim = static_cast<int64_t>(H) * D, C = 3 * dim;
  const int W = T + 2;  // page columns
  const int acc = accepted[b];
  int cslot = 0, src = 0;
  if (acc >= 1 && acc <= T) {
    src = slots[b * cols + acc - 1];
    cslot = slots[b * cols];
  }
  const bool live = src > 0 && cslot > 0 && cslot < pool_slots;
  if (!live) {  // padding: zero outputs, conv state untouched
    const float2 z = make_float2(0.f, 0.f);
    for (int t = 0; t < T; ++t) {
      const int64_t row = (b * T + t) * H + h, out = row * D + c;
      *reinterpret_cast<float2*>(q + out) = z;
      *reinterpret_cast<float2*>(k + out) = z;
      *reinterpret_cast<float2*>(v + out) = z;
      if (c == 0) beta[row] = 0.f;
    }
    return;
  }
  float2 y[3][kMaxT];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int64_t ch = s * dim + static_cast<int64_t>(h) * D + c;
    const float* wc = conv_w + (s * 4) * dim + static_cast<int64_t>(h) * D + c;  // weights [3][4][dim]
    float2 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = *reinterpret_cast<const float2*>(wc + i * dim);
    const float2 bias = BIAS ? *reinterpret_cast<const float2*>(conv_bias + ch) : make_float2(0.f, 0.f);
    __bf16* page0 = conv_state + (static_cast<int64_t>(cslot) * C + ch) * W;  // channel c; c + 1 at + W
    // the window: three taps, then the tokens' inputs
    float s0[kMaxT + 3], s1[kMaxT + 3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      s0[j] = static_cast<float>(page0[acc - 1 + j]);
      s1[j] = static_cast<float>(page0[W + acc - 1 + j]);
    }
    uint32_t xw[kMaxT];
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
      if (t >= T) break;
      xw[t] = *reinterpret_cast<const uint32_t*>(x + (b * T + t) * C + ch);
      s0[3 + t] = bf_lo(xw[t]);
      s1[3 + t] = bf_hi(xw[t]);
    }
    const __bf16 k0a = page0[acc], k0b = page0[acc + 1], k1a = page0[W + acc], k1b = page0[W + acc + 1];
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
      if (t >= T) break;
      float2 a = bias;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a.x = fmaf(w[i].x, s0[t + i], a.x);
        a.y = fmaf(w[i].y, s1[t + i], a.y);
      }
      y[s][t] = make_float2(a.x / (1.f + expf(-a.x)), a.y / (1.f + expf(-a.y)));  // SiLU
    }
    // the page becomes (column a, column a + 1, x_0 .. x_{T-1})
    page0[0] = k0a;
    page0[1] = k0b;
    page0[W] = k1a;
    page0[W + 1] = k1b;
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
      if (t >= T) break;
      page0[2 + t] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(xw[t] & 0xffffu));
      page0[W + 2 + t] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(xw[t] >> 16));
    }
  }
#pragma unroll
  for (int t = 0; t < kMaxT; ++t) {
    if (t >= T) break;
    const int64_t row = (b * T + t) * H + h, out = row * D + c;
    const float nq = row_sum<D>(y[0][t].x * y[0][t].x + y[0][t].y * y[0][t].y);
    const float nk = row_sum<D>(y[1][t].x * y[1][t].x + y[1][t].y * y[1][t].y);
    const float rq = rsqrtf(nq + 1e-6f), rk = rsqrtf(nk + 1e-6f);
    *reinterpret_cast<float2*>(q + out) = make_float2(y[0][t].x * rq, y[0][t].y * rq);
    *reinterpret_cast<float2*>(k + out) = make_float2(y[1][t].x * rk, y[1][t].y * rk);
    *reinterpret_cast<float2*>(v + out) = y[2][t];
    if (c == 0) beta[row] = 1.f / (1.f + expf(-beta_raw[row]));
  }
}

__device__ __forceinline__ void store_pair(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
__device__ __forceinline__ void store_pair(__bf16* p, float a, float b) {
  __bf16 t[2] = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  *reinterpret_cast<uint32_t*>(p) = *reinterpret_cast<const uint32_t*>(t);
}

template <int D, typename Tout>
__global__ __launch_bounds__(kLayerThreads) void gated_rmsnorm_kernel(const float* __restrict__ o,
                                                                      const __bf16* __restrict__ gate,
                                                                      const float* __restrict__ norm_w, float eps,
                                                                      Tout* __restrict__ out, int64_t rows) {
  constexpr int LPH = D / 2;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kLayerThreads + threadIdx.x;
  if (gid / LPH >= rows) return;  // whole rows leave together
  const int c = 2 * static_cast<int>(gid % LPH);
  const int64_t i = 2 * gid;  // element (request, head, c) of the [rows, D] layout
  const float2 x = *reinterpret_cast<const float2*>(o + i);
  const uint32_t gw = *reinterpret_cast<const uint32_t*>(gate + i);
  const float2 w = *reinterpret_cast<const float2*>(norm_w + c);
  const float ss = row_sum<D>(x.x * x.x + x.y * x.y);
  const float r = rsqrtf(ss * (1.f / D) + eps);
  store_pair(out + i, x.x * r * w.x / (1.f + expf(-bf_lo(gw))), x.y * r * w.y / (1.f + expf(-bf_hi(gw))));
}

static unsigned layer_blocks(int64_t rows, int D) {
  return static_cast<unsigned>((rows * (D / 2) + kLayerThreads - 1) / kLayerThreads);
}

hipError_t launch_decode_prologue(const PrologueArgs& a) {
  const int64_t groups = static_cast<int64_t>((a.N + kPrologueReqs - 1) / kPrologueReqs) * a.H;
  const dim3 grid(layer_blocks(groups, a.D));
  auto kern = a.D == 128 ? (a.conv_bias ? decode_prologue_kernel<128, true> : decode_prologue_kernel<128, false>)
                         : (a.conv_bias ? decode_prologue_kernel<64, true> : decode_prologue_kernel<64, false>);
  hipLaunchKernelGGL(kern, grid, dim3(kLayerThreads), 0, a.stream, static_cast<const __bf16*>(a.x), a.conv_w,
                     a.conv_bias, static_cast<__bf16*>(a.conv_state), a.pool_slots, a.slots, a.beta_raw, a.q, a.k,
                     a.v, a.beta, a.N, a.H, groups);
  return hipGetLastError();
}

hipError_t launch_decode_prologue_verify(const PrologueArgs& a) {
  const int64_t groups = static_cast<int64_t>(a.N) * a.H;
  const dim3 grid(layer_blocks(groups, a.D));
  auto kern = a.D == 128 ? (a.conv_bias ? decode_prologue_verify_kernel<128, true>
                                        : decode_prologue_verify_kernel<128, false>)
                         : (a.conv_bias ? decode_prologue_verify_kernel<64, true>
                                        : decode_prologue_verify_kernel<64, false>);
  hipLaunchKernelGGL(kern, grid, dim3(kLayerThreads), 0, a.stream, static_cast<const __bf16*>(a.x), a.conv_w,
                     a.conv_bias, static_cast<__bf16*>(a.conv_state), a.pool_slots, a.slots, a.cols, a.accepted,
                     a.beta_raw, a.q, a.k, a.v, a.beta, a.N, a.T, a.H);
  return hipGetLastError();
}

hipError_t launch_gated_rmsnorm(const RmsNormArgs& a) {
  const int64_t rows = static_cast<int64_t>(a.N) * a.H;
  const dim3 grid(layer_blocks(rows, a.D)), block(kLayerThreads);
  const __bf16* gate = static_cast<const __bf16*>(a.gate);
  if (a.out_f32) {
    auto kern = a.D == 128 ? gated_rmsnorm_kernel<128, float> : gated_rmsnorm_kernel<64, float>;
    hipLaunchKernelGGL(kern, grid, block, 0, a.stream, a.o, gate, a.norm_w, a.eps, static_cast<float*>(a.out), rows);
  } else {
    auto kern = a.D == 128 ? gated_rmsnorm_kernel<128, __bf16> : gated_rmsnorm_kernel<64, __bf16>;
    hipLaunchKernelGGL(kern, grid, block, 0, a.stream, a.o, gate, a.norm_w, a.eps, static_cast<__bf16*>(a.out), rows);
  }
  return hipGetLastError();
}

}  // namespace gdn

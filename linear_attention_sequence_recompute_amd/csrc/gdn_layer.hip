// Front and back operations of the decode layer around the recurrent step (the
// vLLM KdaSplit page, kernel body): before it, a causal depthwise convolution of 4
// taps over the conv-state pool (the slot's last three inputs, then the token's),
// SiLU, the per-head L2 norm of q and k (1e-6 inside the square root) and
// beta = sigmoid(raw beta); after it, the gated RMSNorm of each head's output,
// o * rsqrt(mean(o^2) + eps) * w * sigmoid(gate). That page fuses these steps into
// its decode kernel; here they are two small kernels beside the decode step.
//
// One workgroup per (request, head), one thread per channel of the head (D = 64
// or 128): each thread convolves its channel of the three sections (q, k, v),
// the head's sums of squares go through a wave shuffle and LDS.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

template <int D>
__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  constexpr int W = D / 64 > 0 ? D / 64 : 1;
  if (W == 1) return x;
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < W; ++i) s += red[i];
  return s;
}

template <int D>
__global__ __launch_bounds__(D) void decode_prologue_kernel(
    const __bf16* __restrict__ x, const float* __restrict__ conv_w, const float* __restrict__ conv_bias,
    __bf16* __restrict__ conv_state, int64_t pool_slots, const int32_t* __restrict__ slots,
    const float* __restrict__ beta_raw, float* __restrict__ q, float* __restrict__ k, float* __restrict__ v,
    float* __restrict__ beta, int H) {
  __shared__ float red[2][2];
  const int b = blockIdx.x / H, h = blockIdx.x % H, c = threadIdx.x;
  const int64_t dim = static_cast<int64_t>(H) * D, C = 3 * dim;
  const int64_t out = (static_cast<int64_t>(b) * H + h) * D + c;
  const int slot = slots[b];
  if (slot <= 0 || slot >= pool_slots) {  // padding: zero outputs, conv state untouched
    q[out] = 0.f;
    k[out] = 0.f;
    v[out] = 0.f;
    if (c == 0) beta[static_cast<int64_t>(b) * H + h] = 0.f;
    return;
  }
  float y[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int64_t ch = s * dim + static_cast<int64_t>(h) * D + c;
    __bf16* st = conv_state + (static_cast<int64_t>(slot) * C + ch) * 3;
    const float t0 = static_cast<float>(st[0]), t1 = static_cast<float>(st[1]), t2 = static_cast<float>(st[2]);
    const __bf16 xb = x[static_cast<int64_t>(b) * C + ch];
    const float* wc = conv_w + (s * 4) * dim + static_cast<int64_t>(h) * D + c;  // weights [3][4][dim]
    float acc = conv_bias ? conv_bias[ch] : 0.f;
    acc = fmaf(wc[0], t0, acc);
    acc = fmaf(wc[dim], t1, acc);
    acc = fmaf(wc[2 * dim], t2, acc);
    acc = fmaf(wc[3 * dim], static_cast<float>(xb), acc);
    y[s] = acc / (1.f + expf(-acc));  // SiLU
    st[0] = st[1];
    st[1] = st[2];
    st[2] = xb;
  }
  const float nq = block_sum<D>(y[0] * y[0], red[0]);
  const float nk = block_sum<D>(y[1] * y[1], red[1]);
  q[out] = y[0] * rsqrtf(nq + 1e-6f);
  k[out] = y[1] * rsqrtf(nk + 1e-6f);
  v[out] = y[2];
  if (c == 0) {
    const int64_t bh = static_cast<int64_t>(b) * H + h;
    beta[bh] = 1.f / (1.f + expf(-beta_raw[bh]));
  }
}

template <int D, typename Tout>
__global__ __launch_bounds__(D) void gated_rmsnorm_kernel(const float* __restrict__ o, const __bf16* __restrict__ gate,
                                                          const float* __restrict__ norm_w, float eps,
                                                          Tout* __restrict__ out) {
  __shared__ float red[2];
  const int64_t i = static_cast<int64_t>(blockIdx.x) * D + threadIdx.x;  // (request, head) rows of D
  const float x = o[i];
  const float ss = block_sum<D>(x * x, red);
  const float g = static_cast<float>(gate[i]);
  store_out(out + i, x * rsqrtf(ss * (1.f / D) + eps) * norm_w[threadIdx.x] / (1.f + expf(-g)));
}

hipError_t launch_decode_prologue(const PrologueArgs& a) {
  const dim3 grid(static_cast<unsigned>(a.N) * a.H);
  if (a.D == 128)
    hipLaunchKernelGGL((decode_prologue_kernel<128>), grid, dim3(128), 0, a.stream,
                       static_cast<const __bf16*>(a.x), a.conv_w, a.conv_bias, static_cast<__bf16*>(a.conv_state),
                       a.pool_slots, a.slots, a.beta_raw, a.q, a.k, a.v, a.beta, a.H);
  else
    hipLaunchKernelGGL((decode_prologue_kernel<64>), grid, dim3(64), 0, a.stream, static_cast<const __bf16*>(a.x),
                       a.conv_w, a.conv_bias, static_cast<__bf16*>(a.conv_state), a.pool_slots, a.slots, a.beta_raw,
                       a.q, a.k, a.v, a.beta, a.H);
  return hipGetLastError();
}

hipError_t launch_gated_rmsnorm(const RmsNormArgs& a) {
  const dim3 grid(static_cast<unsigned>(a.N) * a.H);
  if (a.D == 128) {
    if (a.out_f32)
      hipLaunchKernelGGL((gated_rmsnorm_kernel<128, float>), grid, dim3(128), 0, a.stream, a.o,
                         static_cast<const __bf16*>(a.gate), a.norm_w, a.eps, static_cast<float*>(a.out));
    else
      hipLaunchKernelGGL((gated_rmsnorm_kernel<128, __bf16>), grid, dim3(128), 0, a.stream, a.o,
                         static_cast<const __bf16*>(a.gate), a.norm_w, a.eps, static_cast<__bf16*>(a.out));
  } else {
    if (a.out_f32)
      hipLaunchKernelGGL((gated_rmsnorm_kernel<64, float>), grid, dim3(64), 0, a.stream, a.o,
                         static_cast<const __bf16*>(a.gate), a.norm_w, a.eps, static_cast<float*>(a.out));
    else
      hipLaunchKernelGGL((gated_rmsnorm_kernel<64, __bf16>), grid, dim3(64), 0, a.stream, a.o,
                         static_cast<const __bf16*>(a.gate), a.norm_w, a.eps, static_cast<__bf16*>(a.out));
  }
  return hipGetLastError();
}

}  // namespace gdn

// The decode layer in one launch (the vLLM KdaSplit page's kernel body, one token
// per request): causal conv over the conv-state pool + SiLU, per-head q / k L2
// norm and beta = sigmoid(raw), the delta-rule update of the slot's state (a
// scalar decay per token and head, or one per key channel), and the gated
// RMSNorm of the head's output.
//
// One workgroup of 1024 threads per (request, head) holds the head's whole state
// page (D rows of D floats; D / 4 lanes per row, a float4 each), so that the
// head's conv channels, its norms and its output norm need no other workgroup
// (the page uses a cluster per head and shared memory across it for this). The
// state page's loads are issued first; the front operations run while they are
// in flight.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kLayerWG = 1024;

template <int LPR>
__device__ __forceinline__ float lane_group_sum(float x) {
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// Sum over the first n (a multiple of 64, <= 1024) threads' x, returned to every
// thread; red holds 16 floats.
__device__ __forceinline__ float block_sum(float x, float* red, int n) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  if (lane == 0 && tid < n) red[w] = x;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < n / 64; ++i) s += red[i];
  __syncthreads();
  return s;
}

template <int D, bool KDA, bool BIAS, bool NORM, typename Tout>
__global__ __launch_bounds__(kLayerWG) void decode_layer_kernel(
    const __bf16* __restrict__ x, const float* __restrict__ conv_w, const float* __restrict__ conv_bias,
    __bf16* __restrict__ conv_state, int64_t conv_slots, const int32_t* __restrict__ slots,
    const float* __restrict__ beta_raw, const float* __restrict__ g, float* __restrict__ pool, int64_t pool_slots,
    const __bf16* __restrict__ gate, const float* __restrict__ norm_w, float eps, Tout* __restrict__ out, int H,
    float scale) {
  constexpr int LPR = D / 4;                // lanes per state row
  constexpr int RPP = kLayerWG / LPR;       // rows per pass
  constexpr int PASSES = D / RPP;
  static_assert(PASSES >= 1 && D % RPP == 0, "whole passes");
  __shared__ float yq[D], yk[D], yv[D], yo[D];
  __shared__ float red[16];
  int page, part;
  xcd_page_part<1>(blockIdx.x, gridDim.x, page, part);
  const int b = page / H, h = page % H;
  const int tid = threadIdx.x;
  const int col = (tid % LPR) * 4, rsub = tid / LPR;
  const int64_t tok = static_cast<int64_t>(b) * H + h;
  const int slot = slots[b];
  if (slot <= 0 || slot >= pool_slots || slot >= conv_slots) {  // padding: zero outputs, nothing written
    if (tid < D) out[tok * D + tid] = static_cast<Tout>(0.f);
    return;
  }
  float* S = pool + (static_cast<int64_t>(slot) * H + h) * (static_cast<int64_t>(D) * D);
  f32x4 s[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
    s[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (p * RPP + rsub) * D + col));

  // front: thread t < 3 D convolves channel t % D of section t / D (q, k, v) and
  // shifts its conv state (the slot's last three inputs, oldest first)
  const int64_t dim = static_cast<int64_t>(H) * D, C = 3 * dim;
  if (tid < 3 * D) {
    const int sec = tid / D, c = tid % D;
    const int64_t ch = sec * dim + static_cast<int64_t>(h) * D + c;
    __bf16* st = conv_state + (static_cast<int64_t>(slot) * C + ch) * 3;
    const __bf16 t0 = st[0], t1 = st[1], t2 = st[2];
    const __bf16 xv = x[static_cast<int64_t>(b) * C + ch];
    const float* wc = conv_w + (sec * 4) * dim + static_cast<int64_t>(h) * D + c;
    float a = BIAS ? conv_bias[ch] : 0.f;
    a = fmaf(wc[0], static_cast<float>(t0), a);
    a = fmaf(wc[dim], static_cast<float>(t1), a);
    a = fmaf(wc[2 * dim], static_cast<float>(t2), a);
    a = fmaf(wc[3 * dim], static_cast<float>(xv), a);
    const float y = a / (1.f + expf(-a));  // SiLU
    st[0] = t1;
    st[1] = t2;
    st[2] = xv;
    (sec == 0 ? yq : sec == 1 ? yk : yv)[c] = y;
  }
  __syncthreads();
  const float nq = block_sum(tid < D ? yq[tid] * yq[tid] : 0.f, red, D < 64 ? 64 : D);
  const float nk = block_sum(tid < D ? yk[tid] * yk[tid] : 0.f, red, D < 64 ? 64 : D);
  const float rq = rsqrtf(nq + 1e-6f) * scale, rk = rsqrtf(nk + 1e-6f);
  const float bt = 1.f / (1.f + expf(-beta_raw[tok]));

  // the delta-rule update of the page, rows split over the lane groups
  float kk[4], qq[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kk[e] = yk[col + e] * rk;
    qq[e] = yq[col + e] * rq;
  }
  f32x4 decay;
  if constexpr (KDA) {
    const f32x4 lg = *reinterpret_cast<const f32x4*>(g + tok * D + col);
    decay = f32x4{expf(lg[0]), expf(lg[1]), expf(lg[2]), expf(lg[3])};
  } else {
    const float d = expf(g[tok]);
    decay = f32x4{d, d, d, d};
  }
  float dk[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    s[p] *= decay;
    dk[p] = s[p][0] * kk[0] + s[p][1] * kk[1] + s[p][2] * kk[2] + s[p][3] * kk[3];
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) dk[p] = lane_group_sum<LPR>(dk[p]);
  float dq[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const float vn = bt * (yv[p * RPP + rsub] - dk[p]);
#pragma unroll
    for (int e = 0; e < 4; ++e) s[p][e] = fmaf(kk[e], vn, s[p][e]);
    dq[p] = s[p][0] * qq[0] + s[p][1] * qq[1] + s[p][2] * qq[2] + s[p][3] * qq[3];
    __builtin_nontemporal_store(s[p], reinterpret_cast<f32x4*>(S + (p * RPP + rsub) * D + col));
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) dq[p] = lane_group_sum<LPR>(dq[p]);
  if (tid % LPR == 0) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) yo[p * RPP + rsub] = dq[p];
  }
  __syncthreads();

  // the head's output: gated RMSNorm (or the raw output)
  const float o = tid < D ? yo[tid] : 0.f;
  if constexpr (NORM) {
    const float ss = block_sum(o * o, red, D < 64 ? 64 : D);
    if (tid < D) {
      const float r = rsqrtf(ss * (1.f / D) + eps);
      const float gt = static_cast<float>(gate[tok * D + tid]);
      out[tok * D + tid] = static_cast<Tout>(o * r * norm_w[tid] / (1.f + expf(-gt)));
    }
  } else {
    if (tid < D) out[tok * D + tid] = static_cast<Tout>(o);
  }
}

template <int D, typename Tout>
static void launch_layer_d(const LayerArgs& a) {
  const dim3 grid(static_cast<unsigned>(a.N) * a.H);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kLayerWG), 0, a.stream, static_cast<const __bf16*>(a.x), a.conv_w,
                       a.conv_bias, static_cast<__bf16*>(a.conv_state), a.conv_slots, a.slots, a.beta_raw, a.g,
                       a.pool, a.pool_slots, static_cast<const __bf16*>(a.gate), a.norm_w, a.eps,
                       static_cast<Tout*>(a.out), a.H, a.scale);
  };
  const bool bias = a.conv_bias != nullptr, norm = a.norm_w != nullptr;
  if (a.kda) {
    if (bias)
      norm ? go(decode_layer_kernel<D, true, true, true, Tout>) : go(decode_layer_kernel<D, true, true, false, Tout>);
    else
      norm ? go(decode_layer_kernel<D, true, false, true, Tout>) : go(decode_layer_kernel<D, true, false, false, Tout>);
  } else {
    if (bias)
      norm ? go(decode_layer_kernel<D, false, true, true, Tout>) : go(decode_layer_kernel<D, false, true, false, Tout>);
    else
      norm ? go(decode_layer_kernel<D, false, false, true, Tout>)
           : go(decode_layer_kernel<D, false, false, false, Tout>);
  }
}

hipError_t launch_decode_layer(const LayerArgs& a) {
  if (a.D == 128)
    a.out_f32 ? launch_layer_d<128, float>(a) : launch_layer_d<128, __bf16>(a);
  else
    a.out_f32 ? launch_layer_d<64, float>(a) : launch_layer_d<64, __bf16>(a);
  return hipGetLastError();
}

}  // namespace gdn

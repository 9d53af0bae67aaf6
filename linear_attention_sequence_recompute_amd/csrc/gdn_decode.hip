// Recurrent decode step of the gated delta rule over a slot-indexed state pool.
//
// The vLLM KdaSplit page (method update) streams each value row of the state,
// decays it, dots it with k, forms v_new = (v - dot) beta, adds k v_new to the
// row and dots the result with q; rows are independent, so the state is split
// by value rows across lanes and workgroups. Here one scalar decay per token and
// head replaces that page's per-key-channel decays.
//
// Layout on gfx950: a state row of K floats is covered by K/4 lanes holding one
// float4 each (32 lanes for K = 128), so a wave64 updates 2 (K = 128) or 4
// (K = 64) rows at once and reduces its dot products with xor-shuffles inside
// each row's lane group. A workgroup of 256 threads owns 16 rows of one
// (request, head) state page (8 KiB at K = 128) and issues all of its loads
// before any arithmetic. The page is read and written exactly once, with
// non-temporal hints on both: it is not reused by this launch.
//
// The grid runs (head, row group) fastest and the request slowest, so that
// consecutive workgroups stream one slot's state (heads x rows, contiguous in
// the pool) instead of hopping between the scattered slots of consecutive
// requests (measured on the 512-slot pool with random slots: 5.39 TB/s with the
// request fastest, 5.82 TB/s this way; 32 or 64 rows per workgroup and
// temporal loads or stores are slower). The decode step also gives each XCD a
// contiguous range of pages (xcd_page_part: 6.1 TB/s); for the verify step,
// whose writes go to other slots than its reads, that made no difference.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kDecodeRows = 16;  // state rows per workgroup

template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// KDA: g holds a log-decay per key channel ([N, H, K], the KdaSplit page's
// per-column decays); each lane scales its 4 key columns by their own factors.
template <int K, int V, typename Tin, typename Tout, bool KDA = false>
__global__ __launch_bounds__(256) void recurrent_step_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ pool,
    int64_t pool_slots, const int32_t* __restrict__ slots, Tout* __restrict__ o, int H,
    float scale) {
  constexpr int LPR = K / 4;                     // lanes per state row
  constexpr int RPP = 256 / LPR;                 // rows per pass of the workgroup
  constexpr int PASSES = kDecodeRows / RPP;      // passes per workgroup
  constexpr int NP = V / kDecodeRows;  // row groups per head
  int page, part;
  xcd_page_part<NP>(blockIdx.x, gridDim.x / NP, page, part);
  const int b = page / H, h = page % H;
  const int tid = threadIdx.x;
  const int col = (tid % LPR) * 4;
  const int rsub = tid / LPR;
  const int row0 = part * kDecodeRows;
  const int64_t tok = static_cast<int64_t>(b) * H + h;
  Tout* orow = o + tok * V + row0;
  const int slot = slots[b];
  if (slot <= 0 || slot >= pool_slots) {  // padding: zero output, state untouched
    if (tid < kDecodeRows) store_out(orow + tid, 0.f);
    return;
  }
  float* S = pool + (static_cast<int64_t>(slot) * H + h) * (static_cast<int64_t>(V) * K) +
             static_cast<int64_t>(row0) * K;

  f32x4 s[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
    s[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (p * RPP + rsub) * K + col));

  float kk[4], qq[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kk[e] = ld_in(k + tok * K + col + e);
    qq[e] = scale * ld_in(q + tok * K + col + e);
  }
  float vv[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) vv[p] = ld_in(v + tok * V + row0 + p * RPP + rsub);
  f32x4 decay;
  if constexpr (KDA) {
    const f32x4 lg = *reinterpret_cast<const f32x4*>(g + tok * K + col);
    decay = f32x4{expf(lg[0]), expf(lg[1]), expf(lg[2]), expf(lg[3])};
  } else {
    const float d = expf(g[tok]);
    decay = f32x4{d, d, d, d};
  }
  const float bt = beta[tok];

  float dk[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    s[p] *= decay;
    dk[p] = s[p][0] * kk[0] + s[p][1] * kk[1] + s[p][2] * kk[2] + s[p][3] * kk[3];
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) dk[p] = group_sum<LPR>(dk[p]);
  float dq[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const float vn = bt * (vv[p] - dk[p]);
#pragma unroll
    for (int e = 0; e < 4; ++e) s[p][e] = fmaf(kk[e], vn, s[p][e]);
    dq[p] = s[p][0] * qq[0] + s[p][1] * qq[1] + s[p][2] * qq[2] + s[p][3] * qq[3];
    __builtin_nontemporal_store(s[p], reinterpret_cast<f32x4*>(S + (p * RPP + rsub) * K + col));
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) dq[p] = group_sum<LPR>(dq[p]);
  if (tid % LPR == 0) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) store_out(orow + p * RPP + rsub, dq[p]);
  }
}

// Speculative verify (the KdaSplit class docstring, tokens q > 1): request b's T
// tokens (rows b T + t) run in order from the state in slot[b, accepted[b] - 1];
// the state after token t is stored to slot[b, t] when that slot is in (0,
// pool_slots). A request whose source slot is not (or whose accepted count is
// outside [1, cols]) is padding: zero outputs, no writes. The row layout is the
// decode step's, but one workgroup of 1024 threads takes a whole (request, head)
// page, so that each token's state goes out as one contiguous page (5.36 TB/s
// at 96 requests x 4 tokens, against 5.10-5.24 with 16 rows per workgroup); the
// state rows stay in registers across the tokens, each token's inputs loaded
// while the previous token is applied.
constexpr int kMaxVerifyTokens = 8;
constexpr int kVerifyThreads = 1024;

template <int K, int V, typename Tin, typename Tout>
__global__ __launch_bounds__(kVerifyThreads) void recurrent_verify_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ pool,
    int64_t pool_slots, const int32_t* __restrict__ slots, int cols, const int32_t* __restrict__ accepted,
    Tout* __restrict__ o, int T, int H, float scale) {
  constexpr int LPR = K / 4;                    // lanes per state row
  constexpr int RPP = kVerifyThreads / LPR;     // rows per pass of the workgroup
  constexpr int PASSES = V / RPP;               // passes over the page
  static_assert(V % RPP == 0, "whole passes");
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x;
  const int col = (tid % LPR) * 4;
  const int rsub = tid / LPR;
  constexpr int row0 = 0;
  const int64_t page = static_cast<int64_t>(V) * K;
  const int32_t* srow = slots + static_cast<int64_t>(b) * cols;
  const int acc = accepted[b];
  const int src = acc >= 1 && acc <= cols ? srow[acc - 1] : 0;
  if (src <= 0 || src >= pool_slots) {  // padding: zero outputs, nothing written
    if (tid < V)
      for (int t = 0; t < T; ++t) store_out(o + ((static_cast<int64_t>(b) * T + t) * H + h) * V + row0 + tid, 0.f);
    return;
  }
  const float* S = pool + (static_cast<int64_t>(src) * H + h) * page + static_cast<int64_t>(row0) * K;
  f32x4 s[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
    s[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (p * RPP + rsub) * K + col));

  // inputs of one token, loaded one token ahead of their use (two sets live)
  struct TokIn {
    float kk[4], qq[4], vv[PASSES], decay, bt;
    int dst;
  };
  auto load_tok = [&](int t) {
    TokIn r;
    const int64_t tok = (static_cast<int64_t>(b) * T + t) * H + h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r.kk[e] = ld_in(k + tok * K + col + e);
      r.qq[e] = scale * ld_in(q + tok * K + col + e);
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) r.vv[p] = ld_in(v + tok * V + row0 + p * RPP + rsub);
    r.decay = expf(g[tok]);
    r.bt = beta[tok];
    r.dst = srow[t];
    return r;
  };
  TokIn cur = load_tok(0);
#pragma unroll
  for (int t = 0; t < kMaxVerifyTokens; ++t) {
    if (t >= T) break;
    TokIn nxt = cur;
    if (t + 1 < T) nxt = load_tok(t + 1);
    __builtin_amdgcn_sched_barrier(0);  // the next token's loads go out before this token's work
    const int64_t tok = (static_cast<int64_t>(b) * T + t) * H + h;
    float dk[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      s[p] *= cur.decay;
      dk[p] = s[p][0] * cur.kk[0] + s[p][1] * cur.kk[1] + s[p][2] * cur.kk[2] + s[p][3] * cur.kk[3];
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) dk[p] = group_sum<LPR>(dk[p]);
    float dq[PASSES];
    float* D = cur.dst > 0 && cur.dst < pool_slots
                   ? pool + (static_cast<int64_t>(cur.dst) * H + h) * page + static_cast<int64_t>(row0) * K
                   : nullptr;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const float vn = cur.bt * (cur.vv[p] - dk[p]);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[p][e] = fmaf(cur.kk[e], vn, s[p][e]);
      dq[p] = s[p][0] * cur.qq[0] + s[p][1] * cur.qq[1] + s[p][2] * cur.qq[2] + s[p][3] * cur.qq[3];
      if (D) __builtin_nontemporal_store(s[p], reinterpret_cast<f32x4*>(D + (p * RPP + rsub) * K + col));
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) dq[p] = group_sum<LPR>(dq[p]);
    if (tid % LPR == 0) {
      Tout* orow = o + tok * V + row0;
#pragma unroll
      for (int p = 0; p < PASSES; ++p) store_out(orow + p * RPP + rsub, dq[p]);
    }
    cur = nxt;
  }
}

template <int K, int V, typename Tin, typename Tout>
static hipError_t launch_verify_t(const VerifyArgs& a) {
  const dim3 grid(static_cast<unsigned>(a.N) * a.H);  // request slowest
  hipLaunchKernelGGL((recurrent_verify_kernel<K, V, Tin, Tout>), grid, dim3(kVerifyThreads), 0, a.stream,
                     static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                     static_cast<const Tin*>(a.v), a.g, a.beta, a.pool, a.pool_slots, a.slots, a.cols,
                     a.accepted, static_cast<Tout*>(a.o), a.T, a.H, a.scale);
  return hipGetLastError();
}

template <int K, int V>
static hipError_t launch_verify_kv(const VerifyArgs& a) {
  if (a.in_f32) {
    return a.out_f32 ? launch_verify_t<K, V, float, float>(a) : launch_verify_t<K, V, float, __bf16>(a);
  }
  return a.out_f32 ? launch_verify_t<K, V, __bf16, float>(a) : launch_verify_t<K, V, __bf16, __bf16>(a);
}

hipError_t launch_verify(const VerifyArgs& a) {
  if (a.K == 128 && a.V == 128) return launch_verify_kv<128, 128>(a);
  if (a.K == 128 && a.V == 64) return launch_verify_kv<128, 64>(a);
  if (a.K == 64 && a.V == 128) return launch_verify_kv<64, 128>(a);
  return launch_verify_kv<64, 64>(a);
}

template <int K, int V, typename Tin, typename Tout>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const dim3 grid(static_cast<unsigned>(a.N) * a.H * (V / kDecodeRows));  // request slowest
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, a.stream, static_cast<const Tin*>(a.q),
                       static_cast<const Tin*>(a.k), static_cast<const Tin*>(a.v), a.g, a.beta, a.pool,
                       a.pool_slots, a.slots, static_cast<Tout*>(a.o), a.H, a.scale);
  };
  if (a.kda)
    launch(recurrent_step_kernel<K, V, Tin, Tout, true>);
  else
    launch(recurrent_step_kernel<K, V, Tin, Tout, false>);
  return hipGetLastError();
}

template <int K, int V>
static hipError_t launch_decode_kv(const DecodeArgs& a) {
  if (a.in_f32) {
    return a.out_f32 ? launch_decode_t<K, V, float, float>(a) : launch_decode_t<K, V, float, __bf16>(a);
  }
  return a.out_f32 ? launch_decode_t<K, V, __bf16, float>(a) : launch_decode_t<K, V, __bf16, __bf16>(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.K == 128 && a.V == 128) return launch_decode_kv<128, 128>(a);
  if (a.K == 128 && a.V == 64) return launch_decode_kv<128, 64>(a);
  if (a.K == 64 && a.V == 128) return launch_decode_kv<64, 128>(a);
  return launch_decode_kv<64, 64>(a);
}

}  // namespace gdn

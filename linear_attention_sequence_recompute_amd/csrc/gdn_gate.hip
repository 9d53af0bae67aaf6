// The per-key-channel decay ("gate") stage of the KDA decode layer: the
// projection and the log-decay of gdn_gate.h for every (token, head, key
// channel).
//
// One workgroup per (block of kGateGroups x kGateTok tokens, head): the head's
// F_B rows are copied into LDS once and shared by kGateGroups groups of
// threads, one thread per key channel in each; a thread keeps its F_B row in
// registers as float32 and runs kGateTok tokens, whose activations are read once
// per wave into scalar registers. The blocks of a head share an XCD.
#include "gdn_common.h"
#include "gdn_gate.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kGateTok = 8;     // tokens per thread
constexpr int kGateGroups = 4;  // thread groups per workgroup, sharing the head's F_B rows

__device__ __forceinline__ void unpack8(const u32x4& u, float* dst) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dst[2 * i] = __uint_as_float(u[i] << 16);
    dst[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}

template <int K, int MODE>
__global__ __launch_bounds__(K * kGateGroups) void kda_gate_kernel(
    const __bf16* __restrict__ f_a, const __bf16* __restrict__ f_b, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, float lower_bound, float* __restrict__ g, __bf16* __restrict__ raw_out, int N,
    int H) {
  constexpr int R = kGateRank;
  static_assert(K % 64 == 0, "a wave's lanes share one token group");
  constexpr int TPB = kGateTok * kGateGroups;  // tokens per workgroup
  constexpr int SEG = R / 8;                     // 16-byte segments of an F_B row
  __shared__ u32x4 sw[K * SEG];
  // Workgroups are dealt to the 8 XCDs round-robin by id: the token blocks of
  // one head get ids of one residue mod 8, so they share an XCD and its L2,
  // which then serves their common F_B rows (the grid is padded to whole
  // rounds of 8 heads)
  const int n_tb = (N + TPB - 1) / TPB, xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int h = (idx / n_tb) * 8 + xcd, tb = idx % n_tb;
  if (h >= H) return;  // whole workgroup
  // K is a multiple of 64, so a wave's lanes share one group: its token rows
  // are uniform and their activations stay scalar loads
  const int tid = threadIdx.x, f = tid % K, grp = __builtin_amdgcn_readfirstlane(tid / K);
  // The head's F_B rows into LDS, segment s of row r at s ^ (r % SEG): the 16
  // rows a quarter-wave reads together then hit distinct banks.
  const u32x4* src = reinterpret_cast<const u32x4*>(f_b + static_cast<int64_t>(h) * K * R);
  for (int i = tid; i < K * SEG; i += K * kGateGroups) {
    const int r = i / SEG, sg = i % SEG;
    sw[r * SEG + (sg ^ (r % SEG))] = src[i];
  }
  __syncthreads();
  float w[R];
#pragma unroll
  for (int c8 = 0; c8 < SEG; ++c8) unpack8(sw[f * SEG + (c8 ^ (f % SEG))], &w[8 * c8]);
  const int t0 = tb * TPB + grp * kGateTok;
  const int nt = min(kGateTok, N - t0);  // <= 0 for the groups past the last token
  const float ea = expf(a_log[h]);
  const float dt = dt_bias[h * K + f];

  // one token at a time (a wave issues dependent VALU operations back to back;
  // two tokens' chains side by side were slower); the token's activations are
  // the same for every lane: uniform loads, which the compiler places in scalar
  // registers
  for (int t = 0; t < nt; ++t) {
    const uint32_t* xr = reinterpret_cast<const uint32_t*>(f_a) + static_cast<int64_t>(t0 + t) * (R / 2);
    const float raw = gate_raw<MODE>([&](int c) { return bf16_pair_col(xr, c); }, [&](int c) { return w[c]; });
    const __bf16 rg = static_cast<__bf16>(raw);  // round to nearest even
    const int64_t o = (static_cast<int64_t>(t0 + t) * H + h) * K + f;
    g[o] = gate_log_decay(rg, ea, dt, lower_bound);
    if (raw_out) raw_out[o] = rg;
  }
}

template <int K>
static void launch_gate_k(const GateArgs& a) {
  const int64_t n_tb = (a.N + kGateTok * kGateGroups - 1) / (kGateTok * kGateGroups);
  const dim3 grid(static_cast<unsigned>(n_tb * ((a.H + 7) / 8) * 8));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(K * kGateGroups), 0, a.stream, static_cast<const __bf16*>(a.f_a),
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

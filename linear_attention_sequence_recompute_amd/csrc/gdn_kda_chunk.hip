// Chunk form of the delta rule with a decay per key channel (the vLLM KdaSplit
// page, method `update`: every key column of the state decays by its own factor
// before the delta-rule write), over equal-length sequences.
//
// Within a chunk of 64 tokens let G_i be the inclusive cumulative sum of the
// per-channel log-decays (G_i in R^K, non-increasing). With h the [K, V] state at
// the chunk start, the decayed state seen by token i is diag(e^{G_i}) h plus the
// writes of the earlier tokens, each decayed channel by channel from its own
// token on. Writing the chunk's deltas D (rows delta_i) as the unknowns gives
//   (I + L) D = diag(beta) (V - (K o e^G) h),  L_ij = beta_i sum_c k_ic k_jc e^{G_ic - G_jc}  (j < i)
//   o_i = s (q_i o e^{G_i})^T h + sum_{j <= i} P_ij delta_j,  P_ij = s sum_c q_ic k_jc e^{G_ic - G_jc}
//   h' = diag(e^{G_last}) h + (K o e^{G_last - G})^T D
// Every exponent above is <= 0, so nothing overflows. prep forms, per (chunk,
// head), A' = (I + L)^{-1} diag(beta), P and the three scaled K / q operands;
// the scan carries a 16-column slice of h through the chunks of a sequence, its
// products on the fp32 MFMA.
#include "gdn_common.h"
#include "gdn_internal.h"

#include <utility>

namespace gdn {

constexpr int kKdaThreads = 256;  // scan
constexpr int kPrepThreads = 512;  // prep: one workgroup per CU (its LDS), so eight waves

// Four consecutive inputs as float (8-byte loads for bf16, 16-byte for float).
__device__ __forceinline__ float4 ld_in4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld_in4(const __bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}
constexpr float kLog2e = 1.4426950408889634f;

// 2^x by the hardware's v_exp_f32 (about 1 ulp); every argument here is <= 0, and
// results below the normal range become 0, as the exponentials they stand for
// are then negligible against the other terms of their sums.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr int kKdaSlice = 16;  // value columns of the state per scan workgroup

// 16-deep fp32 product on v_mfma_f32_16x16x4f32 with k = 16 kb + 4 g + e in
// instruction e: lane (g, c) supplies a = X[c][16 kb + 4 g + e] and
// b = Y[16 kb + 4 g + e][c], so both come from one 16-byte LDS read each when X
// is stored by rows and Y by columns.
__device__ __forceinline__ f32x4 kda_mma16(const float4& a, const float4& b, f32x4 acc) {
  acc = mfma_f32(a.x, b.x, acc);
  acc = mfma_f32(a.y, b.y, acc);
  acc = mfma_f32(a.z, b.z, acc);
  return mfma_f32(a.w, b.w, acc);
}
__device__ __forceinline__ float4 lds4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// Floats per (chunk, head) in the workspace: A' [64][64], P [64][64], then
// K o e^G, s q o e^G, K o e^{G_last - G} (each [64][K]) and e^{G_last} [K].
__host__ __device__ constexpr int64_t kda_floats_per_chunk(int K) { return 2 * 64 * 64 + 3 * 64 * K + K; }

constexpr float kMinLogDecay = -100.f;  // per token and channel

// Chunk c (global index over the packed sequences) of head h: first token t0 and
// n rows. Packed calls read the schedule (info); an entry that does not fit the
// token stream marks an empty chunk, whose workspace no scan reads.
struct KdaChunkGeo {
  const int4* info;
  int T_eq, ncs_eq, total_tokens;
  __device__ bool at(int c, int& t0, int& n) const {
    if (info) {
      const int4 ci = info[c];
      t0 = ci.y;
      n = ci.z;
      return ci.x >= 0 && n > 0 && n <= 64 && t0 >= 0 && t0 <= total_tokens - n;
    }
    const int s = c / ncs_eq, j = c % ncs_eq;
    t0 = s * T_eq + 64 * j;
    n = min(64, T_eq - 64 * j);
    return n > 0;
  }
};

template <int K, typename Tin>
__global__ __launch_bounds__(kPrepThreads) void kda_prep_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                                                               const float* __restrict__ g,
                                                               const float* __restrict__ beta,
                                                               float* __restrict__ ws, KdaChunkGeo geo, int H,
                                                               float scale) {
  constexpr int LD = K + 4;  // row stride: rows read at the same column fall in different banks
  __shared__ __attribute__((aligned(16))) float sQ[64 * LD];
  __shared__ __attribute__((aligned(16))) float sK[64 * LD];
  __shared__ __attribute__((aligned(16))) float sG[64 * LD];
  __shared__ float sL[64][65];
  __shared__ float sA[64][65];
  __shared__ float sX[16][65];  // the earlier blocks' part of a block row of A
  __shared__ float sB[64];
  const int h = blockIdx.y;
  int t0, n;
  if (!geo.at(blockIdx.x, t0, n)) return;
  const int tid = threadIdx.x;
  float* base = ws + (static_cast<int64_t>(blockIdx.x) * H + h) * kda_floats_per_chunk(K);
  float *Ap = base, *P = base + 4096, *Kg = base + 8192, *Qg = Kg + 64 * K, *Kd = Qg + 64 * K, *gL = Kd + 64 * K;

  // Rows past the sequence end: q = k = 0, g = 0, beta = 0. Every load is issued
  // before the first LDS write, four channels at a time, rows past the end
  // reading the last row (a load under a branch would be waited for at once).
  constexpr int G4 = 64 * K / 4 / kPrepThreads;  // 4-channel groups per lane and operand
  float4 lq[G4], lk[G4], lg[G4];
#pragma unroll
  for (int m = 0; m < G4; ++m) {
    const int e = tid + kPrepThreads * m, i = e / (K / 4), c4 = 4 * (e % (K / 4));
    const int64_t idx = ((static_cast<int64_t>(t0) + min(i, n - 1)) * H + h) * K + c4;
    lq[m] = ld_in4(q + idx);
    lk[m] = ld_in4(k + idx);
    lg[m] = *reinterpret_cast<const float4*>(g + idx);
  }
  const float bt = beta[(static_cast<int64_t>(t0) + min(tid & 63, n - 1)) * H + h];
#pragma unroll
  for (int m = 0; m < G4; ++m) {
    const int e = tid + kPrepThreads * m, i = e / (K / 4), c4 = 4 * (e % (K / 4));
    const float f = i < n ? 1.f : 0.f;  // values, not references, are selected: the arrays stay in registers
    const float fg = f * kLog2e;        // base-2 exponents: e^x = 2^(x log2 e)
    const float4 x = lq[m], y = lk[m], z = lg[m];
    *reinterpret_cast<float4*>(&sQ[i * LD + c4]) = make_float4(f * x.x, f * x.y, f * x.z, f * x.w);
    *reinterpret_cast<float4*>(&sK[i * LD + c4]) = make_float4(f * y.x, f * y.y, f * y.z, f * y.w);
    // a log-decay of -inf (the channel forgets everything) is taken as kMinLogDecay:
    // its factor e^-100 is 0 to every digit that matters, while the differences
    // G_i - G_j of cumulative sums stay finite (-inf - -inf would be NaN)
    *reinterpret_cast<float4*>(&sG[i * LD + c4]) =
        make_float4(fg * fmaxf(z.x, kMinLogDecay), fg * fmaxf(z.y, kMinLogDecay), fg * fmaxf(z.z, kMinLogDecay),
                    fg * fmaxf(z.w, kMinLogDecay));
  }
  if (tid < 64) sB[tid] = tid < n ? bt : 0.f;
  __syncthreads();
  for (int cc = tid; cc < K; cc += kPrepThreads) {  // inclusive cumulative sum over the chunk's tokens
    float s = 0.f;
    for (int i = 0; i < 64; ++i) {
      s += sG[i * LD + cc];
      sG[i * LD + cc] = s;
    }
  }
  __syncthreads();

  // Diagonal 16 x 16 blocks of the pair matrices (j <= i within a block of 16
  // tokens): 4 x 136 pairs spread evenly, one exponent per pair and channel.
  for (int p = tid; p < 4 * 136; p += kPrepThreads) {
    const int blk = p / 136, pp = p % 136;
    int a = static_cast<int>((sqrtf(8.f * pp + 1.f) - 1.f) * 0.5f);
    while ((a + 1) * (a + 2) / 2 <= pp) ++a;
    while (a * (a + 1) / 2 > pp) --a;
    const int i = 16 * blk + a, j = 16 * blk + pp - a * (a + 1) / 2;
    float accP = 0.f, accL = 0.f;
#pragma unroll 4
    for (int cc = 0; cc < K; cc += 4) {
      const float4 qi = *reinterpret_cast<const float4*>(&sQ[i * LD + cc]);
      const float4 ki = *reinterpret_cast<const float4*>(&sK[i * LD + cc]);
      const float4 kj = *reinterpret_cast<const float4*>(&sK[j * LD + cc]);
      const float4 gi = *reinterpret_cast<const float4*>(&sG[i * LD + cc]);
      const float4 gj = *reinterpret_cast<const float4*>(&sG[j * LD + cc]);
      const float e0 = exp2_hw(gi.x - gj.x), e1 = exp2_hw(gi.y - gj.y), e2 = exp2_hw(gi.z - gj.z),
                  e3 = exp2_hw(gi.w - gj.w);
      const float w0 = kj.x * e0, w1 = kj.y * e1, w2 = kj.z * e2, w3 = kj.w * e3;
      accP = fmaf(qi.x, w0, fmaf(qi.y, w1, fmaf(qi.z, w2, fmaf(qi.w, w3, accP))));
      accL = fmaf(ki.x, w0, fmaf(ki.y, w1, fmaf(ki.z, w2, fmaf(ki.w, w3, accL))));
    }
    P[i * 64 + j] = scale * accP;
    if (j < i) sL[i][j] = sB[i] * accL;
  }
  // Off-diagonal blocks (I > J) as fp32 MFMA products: with the reference token
  // r = 16 I between the two blocks, e^{G_i - G_j} = e^{G_i - G_r} e^{G_r - G_j},
  // both factors <= 1, so the rows of block I (q and k) scaled by the first and
  // the rows of block J (k) by the second multiply as plain matrices. Wave w
  // takes block w of (1,0) (2,0) (2,1) (3,0) (3,1) (3,2). Lane (g, c)
  // supplies row c of each operand at channels 16 kb + 4 g .. + 3 and holds rows
  // 4 g .. 4 g + 3, column c of the 16 x 16 results.
  {
    const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
    for (int ob = w; ob < 6; ob += kPrepThreads / 64) {
      const int I = ob < 1 ? 1 : ob < 3 ? 2 : 3, J = ob < 1 ? 0 : ob < 3 ? ob - 1 : ob - 3;
      const int ri = 16 * I + c, rj = 16 * J + c, r0 = 16 * I;
      f32x4 accP = zero4(), accL = zero4();
      for (int kb = 0; kb < K / 16; ++kb) {
        const int cc = 16 * kb + 4 * g;
        const float4 qi = *reinterpret_cast<const float4*>(&sQ[ri * LD + cc]);
        const float4 ki = *reinterpret_cast<const float4*>(&sK[ri * LD + cc]);
        const float4 kj = *reinterpret_cast<const float4*>(&sK[rj * LD + cc]);
        const float4 gi = *reinterpret_cast<const float4*>(&sG[ri * LD + cc]);
        const float4 gj = *reinterpret_cast<const float4*>(&sG[rj * LD + cc]);
        const float4 gr = *reinterpret_cast<const float4*>(&sG[r0 * LD + cc]);
        const float ea[4] = {exp2_hw(gi.x - gr.x), exp2_hw(gi.y - gr.y), exp2_hw(gi.z - gr.z), exp2_hw(gi.w - gr.w)};
        const float eb[4] = {exp2_hw(gr.x - gj.x), exp2_hw(gr.y - gj.y), exp2_hw(gr.z - gj.z), exp2_hw(gr.w - gj.w)};
        const float qa[4] = {qi.x, qi.y, qi.z, qi.w}, ka[4] = {ki.x, ki.y, ki.z, ki.w};
        const float kb4[4] = {kj.x, kj.y, kj.z, kj.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float bv = kb4[e] * eb[e];
          accP = mfma_f32(qa[e] * ea[e], bv, accP);
          accL = mfma_f32(ka[e] * ea[e], bv, accL);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r, j = 16 * J + c;
        P[i * 64 + j] = scale * accP[r];
        sL[i][j] = sB[i] * accL[r];
      }
    }
  }
  __syncthreads();

  if (tid < 64) {
    // A = (I + L)^{-1}, A_ij = delta_ij - sum_{m < i} L_im A_mj (A is unit lower
    // triangular), by blocks of 16 rows on this wave: the part of the sum over
    // the earlier blocks (m < 16 R) is one fp32 MFMA product into sX, the rest
    // a forward substitution within the block, one column per lane. LDS written
    // and read by this one wave needs no barrier: its LDS accesses run in order.
    const int j = tid, g = tid >> 4, c = tid & 15;
    for (int R = 0; R < 4; ++R) {
      if (R > 0) {
        for (int ct = 0; ct < 4; ++ct) {
          f32x4 acc = zero4();
          for (int kb = 0; kb < R; ++kb) {
            const int k0 = 16 * kb + 4 * g, row = 16 * R + c, col = 16 * ct + c;
            acc = kda_mma16(make_float4(sL[row][k0], sL[row][k0 + 1], sL[row][k0 + 2], sL[row][k0 + 3]),
                            make_float4(sA[k0][col], sA[k0 + 1][col], sA[k0 + 2][col], sA[k0 + 3][col]), acc);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) sX[4 * g + r][16 * ct + c] = acc[r];
        }
        __builtin_amdgcn_wave_barrier();
      }
      for (int ii = 0; ii < 16; ++ii) {
        const int i = 16 * R + ii;
        float a0 = R > 0 ? sX[ii][j] : 0.f, a1 = 0.f;
        int m = 16 * R;
        for (; m + 1 < i; m += 2) {
          a0 = fmaf(sL[i][m], sA[m][j], a0);
          a1 = fmaf(sL[i][m + 1], sA[m + 1][j], a1);
        }
        if (m < i) a0 = fmaf(sL[i][m], sA[m][j], a0);
        const float acc = a0 + a1;
        sA[i][j] = i == j ? 1.f : (i > j ? -acc : 0.f);
      }
      __builtin_amdgcn_wave_barrier();
    }
  } else {
    // Meanwhile the other waves write the state-side operands.
    for (int e = tid - 64; e < 64 * K; e += kPrepThreads - 64) {
      const int i = e / K, cc = e % K;
      const float G = sG[i * LD + cc], GL = sG[63 * LD + cc];
      const float eg = exp2_hw(G);
      Kg[e] = sK[i * LD + cc] * eg;
      Qg[e] = scale * sQ[i * LD + cc] * eg;
      Kd[e] = sK[i * LD + cc] * exp2_hw(GL - G);
    }
    for (int cc = tid - 64; cc < K; cc += kPrepThreads - 64) gL[cc] = exp2_hw(sG[63 * LD + cc]);
  }
  __syncthreads();
  for (int e = tid; e < 4096; e += kPrepThreads) {
    const int i = e >> 6, j = e & 63;
    Ap[e] = sA[i][j] * sB[j];  // A' = A diag(beta); zero above the diagonal
    if (j > i) P[e] = 0.f;
  }
}

// Scan operands of one (chunk, head) in LDS: rows padded by 4 floats so that
// the 16 rows one MFMA operand read touches spread over the banks.
template <int K>
struct KdaScanLds {
  static constexpr int LDX = K + 4, LDA = 68, LDT = 68;
  static constexpr int kRowF4 = K / 4;            // float4 per [64][K] row
  static constexpr int kMK = 64 * kRowF4 / 256;   // prefetch steps per [64][K] operand
  static constexpr int kSteps = 8 + 3 * kMK + 1;  // A', P (4 steps each), three [64][K], e^{G_last}
  float Kg[64 * LDX], Qg[64 * LDX];
  float Kd[64 * LDX];  // K o e^{G_last - G}
  float Ap[64 * LDA], P[64 * LDA];
  float gL[K];
  float hT[16 * LDX];  // the state slice, transposed: [value column][key]
  float RT[16 * LDT];  // (V - (K o e^G) h)^T
  float DT[16 * LDT];  // the chunk's deltas, transposed
};


// The chunk's workspace block, float4 f = tid + 256 m, loaded into registers:
// steps [0, kHalf) in one array and the rest in another (two arrays of this size
// stay in registers where one of the whole size is placed in scratch memory).
template <int K>
struct KdaPf {
  static constexpr int kHalf = KdaScanLds<K>::kSteps / 2;
  float4 a[kHalf];
  float4 b[KdaScanLds<K>::kSteps - kHalf];
};

template <int K, int M>
__device__ __forceinline__ float4 kda_ld(const float4* s4, int tid) {
  using L = KdaScanLds<K>;
  return M < L::kSteps - 1 ? s4[tid + 256 * M] : s4[min(tid, K / 4 - 1) + 256 * M];  // last: e^{G_last}, no branch
}

template <int K, int M>
__device__ __forceinline__ void kda_st(const float4& x, KdaScanLds<K>& sm, int tid) {
  using L = KdaScanLds<K>;
  if constexpr (M == L::kSteps - 1) {
    if (tid < K / 4) *reinterpret_cast<float4*>(&sm.gL[4 * tid]) = x;
  } else {
    float* dst;
    if constexpr (M < 8) {
      const int f = tid + 256 * (M & 3);
      dst = (M < 4 ? sm.Ap : sm.P) + (f >> 4) * L::LDA + 4 * (f & 15);
    } else {
      constexpr int op = (M - 8) / L::kMK;
      const int f = tid + 256 * ((M - 8) % L::kMK);
      const int row = f / L::kRowF4, col = 4 * (f % L::kRowF4);
      dst = (op == 0 ? sm.Kg : op == 1 ? sm.Qg : sm.Kd) + row * L::LDX + col;
    }
    *reinterpret_cast<float4*>(dst) = x;
  }
}

template <int K, int... Ms>
__device__ __forceinline__ void kda_prefetch_seq(KdaPf<K>& pf, const float4* s4, int tid,
                                                 std::integer_sequence<int, Ms...>) {
  constexpr int h = KdaPf<K>::kHalf;
  ((Ms < h ? (void)(pf.a[Ms < h ? Ms : 0] = kda_ld<K, Ms>(s4, tid))
           : (void)(pf.b[Ms < h ? 0 : Ms - h] = kda_ld<K, Ms>(s4, tid))), ...);
}
template <int K, int... Ms>
__device__ __forceinline__ void kda_stage_seq(const KdaPf<K>& pf, KdaScanLds<K>& sm, int tid,
                                              std::integer_sequence<int, Ms...>) {
  constexpr int h = KdaPf<K>::kHalf;
  ((Ms < h ? kda_st<K, Ms>(pf.a[Ms < h ? Ms : 0], sm, tid) : kda_st<K, Ms>(pf.b[Ms < h ? 0 : Ms - h], sm, tid)),
   ...);
}
template <int K>
__device__ __forceinline__ void kda_prefetch(KdaPf<K>& pf, const float* src, int tid) {
  kda_prefetch_seq<K>(pf, reinterpret_cast<const float4*>(src), tid,
                      std::make_integer_sequence<int, KdaScanLds<K>::kSteps>{});
}
// Steps [M0, M0 + N) only.
template <int K, int M0, int... Ns>
__device__ __forceinline__ void kda_prefetch_part_seq(KdaPf<K>& pf, const float4* s4, int tid,
                                                      std::integer_sequence<int, Ns...>) {
  kda_prefetch_seq<K>(pf, s4, tid, std::integer_sequence<int, (M0 + Ns)...>{});
}
template <int K, int M0, int N>
__device__ __forceinline__ void kda_prefetch_part(KdaPf<K>& pf, const float* src, int tid) {
  kda_prefetch_part_seq<K, M0>(pf, reinterpret_cast<const float4*>(src), tid, std::make_integer_sequence<int, N>{});
}
template <int K>
__device__ __forceinline__ void kda_stage(const KdaPf<K>& pf, KdaScanLds<K>& sm, int tid) {
  kda_stage_seq<K>(pf, sm, tid, std::make_integer_sequence<int, KdaScanLds<K>::kSteps>{});
}

// One workgroup (4 waves) per (value slice of 16 columns, head, sequence); the
// slice of the state (K keys x 16 columns, stored by column) stays in LDS across
// the sequence's chunks. All four products of a chunk run on
// v_mfma_f32_16x16x4f32 (fp32 in, fp32 out) in 16-deep blocks (kda_mma16); each
// lane holds rows 4 g .. 4 g + 3, column c of a 16 x 16 result. Wave w owns
// token rows 16 w .. 16 w + 15 of R, D and o, and K / 64 of the state's 16-key
// tiles. The next chunk's operands are loaded into registers while this one is
// computed.
// Arguments of the scan: the sequences (packed with cu_seqlens and the chunk
// schedule, or of equal length T_eq) and where their states live.
struct KdaScanArgs {
  const float* h0;  // may alias ht (in place)
  float* ht;
  float* pool;
  int64_t pool_slots;
  const int32_t* slots;
  int H, V, n_seqs, T_eq, ncs_eq, total_tokens, n_chunks;
  const int32_t* cu;
  const int* seq_chunk0;
};

template <int K, typename Tin, typename Tout>
__global__ __launch_bounds__(kKdaThreads) void kda_scan_kernel(const Tin* __restrict__ v, const float* __restrict__ ws,
                                                               Tout* __restrict__ o, KdaScanArgs a) {
  using L = KdaScanLds<K>;
  __shared__ __attribute__((aligned(16))) L sm;
  const int H = a.H, V = a.V;
  // Workgroups are dealt to the 8 XCDs round-robin by id: the slices of one
  // (sequence, head) pair get ids of one residue mod 8, so they share an XCD and
  // its L2, which then serves their common reads of the chunk operands.
  const int n_slices = V / kKdaSlice, xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int pair = (idx / n_slices) * 8 + xcd;
  if (pair >= a.n_seqs * H) return;  // padding of the grid to whole rounds of 8
  const int h = pair % H, seq = pair / H;
  // the sequence's tokens and chunks (a packed call whose offsets do not fit the
  // token stream or the chunk count gets an empty sequence)
  int start, len, chunk0;
  if (a.cu) {
    start = a.cu[seq];
    len = a.cu[seq + 1] - start;
    chunk0 = a.seq_chunk0[seq];
    if (start < 0 || len < 0 || start > a.total_tokens - len || chunk0 < 0 ||
        chunk0 > a.n_chunks - (len + 63) / 64)
      len = 0;
  } else {
    start = seq * a.T_eq;
    len = a.T_eq;
    chunk0 = seq * a.ncs_eq;
  }
  const int NC = (len + 63) / 64;
  const int v_base = (idx % n_slices) * kKdaSlice;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  // the state pages: a pool slot (<= 0 or past the pool: zero start, no write) or h0 / ht
  const int64_t page = static_cast<int64_t>(V) * K;
  const float* st_in = nullptr;
  float* st_out = nullptr;
  if (a.pool) {
    const int sl = a.slots[seq];
    if (sl > 0 && sl < a.pool_slots) {
      st_in = a.pool + (static_cast<int64_t>(sl) * H + h) * page;
      st_out = a.pool + (static_cast<int64_t>(sl) * H + h) * page;
    }
  } else {
    if (a.h0) st_in = a.h0 + (static_cast<int64_t>(seq) * H + h) * page;
    if (a.ht) st_out = a.ht + (static_cast<int64_t>(seq) * H + h) * page;
  }
  const int64_t st_row = static_cast<int64_t>(v_base) * K;  // this slice's rows [.., V, K]
  for (int e = tid; e < K * kKdaSlice; e += kKdaThreads) {
    const int cc = e % K, vv = e / K;
    sm.hT[vv * L::LDX + cc] = st_in ? st_in[st_row + vv * K + cc] : 0.f;
  }
  const int64_t per = kda_floats_per_chunk(K);
  const float* ws_bh = ws + (static_cast<int64_t>(chunk0) * H + h) * per;  // chunk c at + c * H * per
  // The next chunk's operands, loaded while this one is computed.
  KdaPf<K> pf;
  Tin vr[4];
  auto load_v = [&](int ch) __attribute__((always_inline)) {  // lane's V values: rows 16 w + 4 g + r, column c
    const int t0 = ch * 64, n = min(64, len - t0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // Rows past the end read the last row and are zeroed where used: a load
      // under a branch would be waited for at once, and with it the prefetch.
      const int ic = min(16 * w + 4 * g + r, n - 1);
      vr[r] = v[((static_cast<int64_t>(start) + t0 + ic) * H + h) * V + v_base + c];
    }
  };
  if (NC > 0) {
    kda_prefetch<K>(pf, ws_bh, tid);
    load_v(0);
  }
  for (int ch = 0; ch < NC; ++ch) {
    const int t0 = ch * 64, n = min(64, len - t0);
    __syncthreads();  // the previous chunk is done with the operands and the state
    kda_stage<K>(pf, sm, tid);
    float vcur[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) vcur[r] = 16 * w + 4 * g + r < n ? ld_in(&vr[r]) : 0.f;
    // The next chunk's operands are loaded in four groups spread over this
    // chunk's steps, each after its registers have been staged above (the last
    // chunk reloads itself, unused: unconditional loads keep pf in registers).
    const float* nxt = ws_bh + static_cast<int64_t>(min(ch + 1, NC - 1)) * H * per;
    constexpr int kKd0 = 8 + 2 * L::kMK;
    kda_prefetch_part<K, kKd0, L::kMK + 1>(pf, nxt, tid);  // K-decay and e^{G_last}
    load_v(min(ch + 1, NC - 1));
    __syncthreads();
    kda_prefetch_part<K, 0, 8>(pf, nxt, tid);  // A', P
    // R = V - (K o e^G) h
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < K / 16; ++kb)
      acc = kda_mma16(lds4(&sm.Kg[(16 * w + c) * L::LDX + 16 * kb + 4 * g]), lds4(&sm.hT[c * L::LDX + 16 * kb + 4 * g]),
                      acc);
    *reinterpret_cast<float4*>(&sm.RT[c * L::LDT + 16 * w + 4 * g]) =
        make_float4(vcur[0] - acc[0], vcur[1] - acc[1], vcur[2] - acc[2], vcur[3] - acc[3]);
    __syncthreads();
    kda_prefetch_part<K, 8, L::kMK>(pf, nxt, tid);  // K o e^G
    // D = A' R (A' vanishes above the diagonal: k < 16 (w + 1))
    acc = zero4();
    for (int kb = 0; kb <= w; ++kb)
      acc = kda_mma16(lds4(&sm.Ap[(16 * w + c) * L::LDA + 16 * kb + 4 * g]), lds4(&sm.RT[c * L::LDT + 16 * kb + 4 * g]),
                      acc);
    *reinterpret_cast<float4*>(&sm.DT[c * L::LDT + 16 * w + 4 * g]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    kda_prefetch_part<K, 8 + L::kMK, L::kMK>(pf, nxt, tid);  // s q o e^G
    // o = (s q o e^G) h + P D
    acc = zero4();
#pragma unroll
    for (int kb = 0; kb < K / 16; ++kb)
      acc = kda_mma16(lds4(&sm.Qg[(16 * w + c) * L::LDX + 16 * kb + 4 * g]), lds4(&sm.hT[c * L::LDX + 16 * kb + 4 * g]),
                      acc);
    for (int kb = 0; kb <= w; ++kb)
      acc = kda_mma16(lds4(&sm.P[(16 * w + c) * L::LDA + 16 * kb + 4 * g]), lds4(&sm.DT[c * L::LDT + 16 * kb + 4 * g]),
                      acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * w + 4 * g + r;
      if (i < n) store_out(o + ((static_cast<int64_t>(start) + t0 + i) * H + h) * V + v_base + c, acc[r]);
    }
    __syncthreads();  // every wave has read the state
    // h' = diag(e^{G_last}) h + (K o e^{G_last - G})^T D, 16 keys at a time:
    // lane (g, c) holds keys 16 t + 4 g + r of value column c
#pragma unroll
    for (int u = 0; u < K / 64; ++u) {
      const int t = w * (K / 64) + u;
      float* hp = &sm.hT[c * L::LDX + 16 * t + 4 * g];
      const float4 h4 = lds4(hp), g4 = lds4(&sm.gL[16 * t + 4 * g]);
      f32x4 hs = f32x4{g4.x * h4.x, g4.y * h4.y, g4.z * h4.z, g4.w * h4.w};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        // a = (K o e^{G_last - G})^T: a column of the row-major tile, four
        // reads that fall in 64 different banks (row stride K + 4)
        const float* kd = &sm.Kd[(16 * kb + 4 * g) * L::LDX + 16 * t + c];
        hs = kda_mma16(make_float4(kd[0], kd[L::LDX], kd[2 * L::LDX], kd[3 * L::LDX]),
                       lds4(&sm.DT[c * L::LDT + 16 * kb + 4 * g]), hs);
      }
      *reinterpret_cast<float4*>(hp) = make_float4(hs[0], hs[1], hs[2], hs[3]);
    }
  }
  __syncthreads();
  if (st_out)
    for (int e = tid; e < K * kKdaSlice; e += kKdaThreads) {
      const int cc = e % K, vv = e / K;
      st_out[st_row + vv * K + cc] = sm.hT[vv * L::LDX + cc];
    }
}

// Workspace: the chunk operands per (chunk, head), then the chunk schedule of
// a packed call (16 bytes per chunk, 4 per sequence and one more).
static size_t kda_ops_bytes(int64_t max_chunks, int H, int K) {
  return (static_cast<size_t>(max_chunks) * H * kda_floats_per_chunk(K) * 4 + 255) & ~static_cast<size_t>(255);
}
size_t kda_workspace_bytes(int64_t max_chunks, int n_seqs, int H, int K) {
  return kda_ops_bytes(max_chunks, H, K) + static_cast<size_t>(max_chunks) * 16 +
         static_cast<size_t>(n_seqs + 1) * 4;
}

template <int K, typename Tin>
static void launch_kda_typed(const KdaChunkArgs& a) {
  const bool varlen = a.cu_seqlens != nullptr;
  const int ncs_eq = varlen ? 0 : (a.T_eq + 63) / 64;
  float* ops = static_cast<float*>(a.ws);
  char* sched = static_cast<char*>(a.ws) + kda_ops_bytes(a.n_chunks, a.H, K);
  int4* info = reinterpret_cast<int4*>(sched);
  int* seq_chunk0 = reinterpret_cast<int*>(sched + a.n_chunks * 16);
  if (varlen)
    (void)launch_chunk_schedule(a.cu_seqlens, a.n_seqs, static_cast<int>(a.total_tokens),
                                static_cast<int>(a.n_chunks), seq_chunk0, info, a.stream);
  if (a.n_chunks > 0)
    hipLaunchKernelGGL((kda_prep_kernel<K, Tin>), dim3(static_cast<unsigned>(a.n_chunks), a.H), dim3(kPrepThreads), 0,
                       a.stream, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), a.g, a.beta, ops,
                       KdaChunkGeo{varlen ? info : nullptr, a.T_eq, ncs_eq, static_cast<int>(a.total_tokens)}, a.H,
                       a.scale);
  if (a.events[1]) (void)hipEventRecord(a.events[1], a.stream);
  KdaScanArgs sa{a.h0, a.ht, a.pool, a.pool_slots, a.slots, a.H, a.V, a.n_seqs, a.T_eq, ncs_eq,
                 static_cast<int>(a.total_tokens), static_cast<int>(a.n_chunks), a.cu_seqlens, seq_chunk0};
  const int64_t n_pairs = static_cast<int64_t>(a.n_seqs) * a.H;
  const dim3 grid(static_cast<unsigned>((n_pairs + 7) / 8) * 8 * (a.V / kKdaSlice));
  if (a.out_f32)
    hipLaunchKernelGGL((kda_scan_kernel<K, Tin, float>), grid, dim3(kKdaThreads), 0, a.stream,
                       static_cast<const Tin*>(a.v), ops, static_cast<float*>(a.o), sa);
  else
    hipLaunchKernelGGL((kda_scan_kernel<K, Tin, __bf16>), grid, dim3(kKdaThreads), 0, a.stream,
                       static_cast<const Tin*>(a.v), ops, static_cast<__bf16*>(a.o), sa);
}

hipError_t launch_chunk_fwd_kda(const KdaChunkArgs& a) {
  if (a.events[0]) (void)hipEventRecord(a.events[0], a.stream);
  if (a.K == 128)
    a.in_f32 ? launch_kda_typed<128, float>(a) : launch_kda_typed<128, __bf16>(a);
  else
    a.in_f32 ? launch_kda_typed<64, float>(a) : launch_kda_typed<64, __bf16>(a);
  if (a.events[2]) (void)hipEventRecord(a.events[2], a.stream);
  return hipGetLastError();
}

}  // namespace gdn

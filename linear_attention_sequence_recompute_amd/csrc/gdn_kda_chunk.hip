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

#include <type_traits>
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

// The (sequence, head, value slice) a scan workgroup serves, and its sequence's
// tokens and chunks. Workgroups are dealt to the 8 XCDs round-robin by id: the
// slices of one (sequence, head) pair get ids of one residue mod 8, so they
// share an XCD and its L2, which serves their common reads of the chunk operands.
struct KdaSeq {
  int seq, h, start, len, chunk0, v_base;
};
__device__ __forceinline__ bool kda_seq_of(const KdaScanArgs& a, KdaSeq& s) {
  const int n_slices = a.V / kKdaSlice, xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int pair = (idx / n_slices) * 8 + xcd;
  if (pair >= a.n_seqs * a.H) return false;  // padding of the grid to whole rounds of 8
  s.h = pair % a.H;
  s.seq = pair / a.H;
  s.v_base = (idx % n_slices) * kKdaSlice;
  // a packed call whose offsets do not fit the token stream or the chunk count
  // gets an empty sequence
  if (a.cu) {
    s.start = a.cu[s.seq];
    s.len = a.cu[s.seq + 1] - s.start;
    s.chunk0 = a.seq_chunk0[s.seq];
    if (s.start < 0 || s.len < 0 || s.start > a.total_tokens - s.len || s.chunk0 < 0 ||
        s.chunk0 > a.n_chunks - (s.len + 63) / 64)
      s.len = 0;
  } else {
    s.start = s.seq * a.T_eq;
    s.len = a.T_eq;
    s.chunk0 = s.seq * a.ncs_eq;
  }
  return true;
}
// The state pages: a pool slot (<= 0 or past the pool: zero start, no write) or h0 / ht.
template <int K>
__device__ __forceinline__ void kda_pages(const KdaScanArgs& a, const KdaSeq& s, const float*& st_in, float*& st_out) {
  const int64_t page = static_cast<int64_t>(a.V) * K;
  st_in = nullptr;
  st_out = nullptr;
  if (a.pool) {
    const int sl = a.slots[s.seq];
    if (sl > 0 && sl < a.pool_slots) {
      st_in = a.pool + (static_cast<int64_t>(sl) * a.H + s.h) * page;
      st_out = a.pool + (static_cast<int64_t>(sl) * a.H + s.h) * page;
    }
  } else {
    if (a.h0) st_in = a.h0 + (static_cast<int64_t>(s.seq) * a.H + s.h) * page;
    if (a.ht) st_out = a.ht + (static_cast<int64_t>(s.seq) * a.H + s.h) * page;
  }
}


template <int K, typename Tin, typename Tout>
__global__ __launch_bounds__(kKdaThreads) void kda_scan_kernel(const Tin* __restrict__ v, const float* __restrict__ ws,
                                                               Tout* __restrict__ o, KdaScanArgs a) {
  using L = KdaScanLds<K>;
  __shared__ __attribute__((aligned(16))) L sm;
  KdaSeq sq;
  if (!kda_seq_of(a, sq)) return;
  const int H = a.H, V = a.V, h = sq.h, start = sq.start, len = sq.len, chunk0 = sq.chunk0, v_base = sq.v_base;
  const int NC = (len + 63) / 64;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const float* st_in;
  float* st_out;
  kda_pages<K>(a, sq, st_in, st_out);
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

// ---------------------------------------------------------------------------
// bf16 inputs: the chunk step on the bf16 MFMA (v_mfma_f32_16x16x32_bf16).
// Every operand of the scan is a computed fp32 matrix (the decays differ per key
// channel, so no product has an exact bf16 side as in the scalar-decay path);
// each is carried as a split bf16 pair hi + lo and each product takes the three
// MFMA terms of two split operands, about 16 significant bits (the same as
// every computed operand of the scalar-decay path).
//
// prep writes, per (chunk, head), the scan's operands as fragments in the
// layout of gdn_common.h (planes of 64 lanes x 16 bytes, hi then lo):
//   kg  [4 row tiles][K/32 key blocks]  K o e^G            (A operand: token rows)
//   qg  [4][K/32]                       s q o e^G
//   kdt [K/16 key tiles][2 token blocks] (K o e^{G_last - G})^T (A operand: key rows)
//   af  [6]                             A' = (I + L)^{-1} diag(beta), nonzero tiles
//   pf  [6]                             P, the same tiles
//   gl  [K] f32                         e^{G_last}
// ---------------------------------------------------------------------------
template <int K>
struct KdaOps {
  static constexpr int NKB = K / 32, NT = K / 16;
  static constexpr int kFrag = 2 * 1024;  // one split fragment: hi plane, lo plane
  static constexpr int kg = 0;
  static constexpr int qg = kg + 4 * NKB * kFrag;
  static constexpr int kdt = qg + 4 * NKB * kFrag;
  static constexpr int af = kdt + NT * 2 * kFrag;
  static constexpr int pf = af + 6 * kFrag;
  static constexpr int gl = pf + 6 * kFrag;
  static constexpr int bytes = (gl + 4 * K + 255) & ~255;
};
static_assert(KdaOps<128>::bytes <= kda_floats_per_chunk(128) * 4, "split operands fit the fp32 layout's space");
static_assert(KdaOps<64>::bytes <= kda_floats_per_chunk(64) * 4, "split operands fit the fp32 layout's space");

// Nonzero A' / P tiles (row tile rt, token block ks): (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).
__device__ __forceinline__ constexpr int kda_a_tile(int rt, int ks) { return rt < 2 ? rt : 2 * rt - 2 + ks; }

// The 8 values at channels c0 + kappa(g, e) of a row, as floats.
__device__ __forceinline__ void kda_row8(const __bf16* row, int c0, int g, float (&x)[8]) {
  const u32x2 a = *reinterpret_cast<const u32x2*>(row + c0 + 4 * g);
  const u32x2 b = *reinterpret_cast<const u32x2*>(row + c0 + 16 + 4 * g);
  const uint32_t u[4] = {a[0], a[1], b[0], b[1]};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(u[e] << 16);
    x[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
  }
}
__device__ __forceinline__ void kda_row8(const float* row, int c0, int g, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(row + c0 + 4 * g);
  const f32x4 b = *reinterpret_cast<const f32x4*>(row + c0 + 16 + 4 * g);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[4 + e] = b[e];
  }
}

// 16-deep fp32 product of two LDS-resident 16 x 16 blocks (v_mfma_f32_16x16x4f32):
// lane (g, c) supplies a = X[c][4 g + e], b = Y[4 g + e][c] to instruction e.
__device__ __forceinline__ f32x4 kda_mma16v(const f32x4& a, const f32x4& b, f32x4 acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = mfma_f32(a[e], b[e], acc);
  return acc;
}

// A diagonal 16 x 16 block of L and P is factored about its middle token m,
// e^{G_i - G_j} = e^{G_i - G_m} e^{G_m - G_j}, when no channel's G moves by more
// than kDiagSpan (log2 units) from G_m within the block, so that neither factor
// leaves the float range; otherwise it is summed pair by pair.
constexpr float kDiagSpan = 64.f;

template <int K>
__global__ __launch_bounds__(256) void kda_prep_split_kernel(const __bf16* __restrict__ q,
                                                             const __bf16* __restrict__ k,
                                                             const float* __restrict__ g,
                                                             const float* __restrict__ beta, char* __restrict__ ws,
                                                             KdaChunkGeo geo, int H, float scale) {
  using P = Prec<__bf16>;
  using Ops = KdaOps<K>;
  constexpr int NKB = K / 32, TPW = K / 64;
  constexpr int LDK = K + 8, LDG = K + 4, LDA = 68;
  constexpr int CQ = K / 4, RG = 256 / CQ, RPG = 64 / RG;  // cumsum: channel quads x row groups
  __shared__ __attribute__((aligned(16))) __bf16 sK[64 * LDK];
  __shared__ __attribute__((aligned(16))) float sG[64 * LDG];  // G log2(e), chunk-local inclusive cumsum
  __shared__ __attribute__((aligned(16))) float sLA[64][LDA];  // L; diagonal blocks become their inverses
  __shared__ float sOff[6][16][17];                             // A_ij below the diagonal
  __shared__ float sB[64];
  const int h = blockIdx.y;
  int t0, n;
  if (!geo.at(blockIdx.x, t0, n)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, lc = lane & 15;
  char* ops = ws + (static_cast<int64_t>(blockIdx.x) * H + h) * Ops::bytes;
  const int64_t rs = static_cast<int64_t>(H) * K;
  const int64_t base = (static_cast<int64_t>(t0) * H + h) * K;
  auto q_row = [&](int i) { return q + base + min(i, n - 1) * rs; };  // rows past the end: masked by the caller
  auto off_block = [](int i, int j) { return i * (i - 1) / 2 + j; };  // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)

  // (0) K into LDS (rows past the end zero), the chunk-local inclusive cumsum of
  // the log-decays into sG by row groups (group totals through sLA), beta
  {
    const int cq = tid % CQ, rg = tid / CQ;
    u32x2 kk[RPG];
    f32x4 gv[RPG];
#pragma unroll
    for (int ii = 0; ii < RPG; ++ii) {
      const int64_t idx = base + min(rg * RPG + ii, n - 1) * rs + 4 * cq;
      kk[ii] = *reinterpret_cast<const u32x2*>(k + idx);
      gv[ii] = *reinterpret_cast<const f32x4*>(g + idx);
    }
    const float bt = tid < 64 ? beta[(static_cast<int64_t>(t0) + min(tid, n - 1)) * H + h] : 0.f;
    f32x4 s = zero4();
#pragma unroll
    for (int ii = 0; ii < RPG; ++ii) {
      const int i = rg * RPG + ii;
      const bool in = i < n;
      const float f = in ? kLog2e : 0.f;
      // a log-decay of -inf is taken as kMinLogDecay (see the fp32 prep)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] += f * fmaxf(gv[ii][e], kMinLogDecay);
      gv[ii] = s;
      *reinterpret_cast<u32x2*>(&sK[i * LDK + 4 * cq]) = in ? kk[ii] : u32x2{0u, 0u};
    }
    float* tot = &sLA[0][0];  // [RG][K]
    *reinterpret_cast<f32x4*>(&tot[rg * K + 4 * cq]) = s;
    if (tid < 64) sB[tid] = tid < n ? bt : 0.f;
    __syncthreads();
    f32x4 off = zero4();
    for (int r2 = 0; r2 < rg; ++r2) off += *reinterpret_cast<const f32x4*>(&tot[r2 * K + 4 * cq]);
#pragma unroll
    for (int ii = 0; ii < RPG; ++ii) *reinterpret_cast<f32x4*>(&sG[(rg * RPG + ii) * LDG + 4 * cq]) = gv[ii] + off;
    __syncthreads();
  }

  // (1) L = StrictLower(diag(beta) ((K o e^G)(K o e^-G)^T)) and P = s (Q o e^G)(K o
  // e^-G)^T masked to j <= i, by 16 x 16 blocks (I, J <= I), grouped into the P
  // fragments (row tile I, token block ks) as in the scalar-decay prep: three,
  // three, two and two blocks per wave. A block below the diagonal is factored
  // about the first token r = 16 I of row block I (both factors <= 1). Each block
  // is computed transposed, (rows j) x (columns i), so that lane (g, c) ends with
  // row i = 16 I + c at the four columns j = 16 J + 4 g + r: a pair of such tiles
  // is one A-operand fragment of P, and L goes to LDS row by row.
  constexpr int kGrp[4][2] = {{0, 6}, {2, 5}, {4, -1}, {7, -1}};
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int grp = kGrp[w][gi];
    if (grp < 0) continue;
    const int I = grp >> 1, ks = grp & 1;
    const int i = 16 * I + lc;
    const float bi = sB[i];
    const float qm = i < n ? scale : 0.f;
    const __bf16* qi_row = q_row(i);
    f32x4 pt[2] = {zero4(), zero4()};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int J = 2 * ks + half;
      if (J > I) continue;
      const int jr = 16 * J + lc;  // the row this lane supplies to the A operand
      bool exact = false;
      int ref = 16 * I;
      if (J == I) {
        ref = 16 * I + 8;
        bool bad = false;
        for (int ch = lane; ch < K; ch += 64) {
          const float gm = sG[ref * LDG + ch];
          bad |= sG[16 * I * LDG + ch] - gm > kDiagSpan || gm - sG[(16 * I + 15) * LDG + ch] > kDiagSpan;
        }
        exact = __ballot(bad) != 0ull;
      }
      f32x4 lacc = zero4(), pacc = zero4();
      if (!exact) {
        f32x4 la[3] = {zero4(), zero4(), zero4()}, pa[3] = {zero4(), zero4(), zero4()};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          float gr[8], kj[8], gj[8], ki[8], gi8[8], qi[8];
          kda_row8(sG + ref * LDG, 32 * kb, lg, gr);
          kda_row8(sK + jr * LDK, 32 * kb, lg, kj);
          kda_row8(sG + jr * LDG, 32 * kb, lg, gj);
          kda_row8(sK + i * LDK, 32 * kb, lg, ki);
          kda_row8(sG + i * LDG, 32 * kb, lg, gi8);
          kda_row8(qi_row, 32 * kb, lg, qi);
          float xa[8], xk[8], xq[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            xa[e] = kj[e] * exp2_hw(gr[e] - gj[e]);
            const float ei = exp2_hw(gi8[e] - gr[e]);
            xk[e] = ki[e] * ei;
            xq[e] = qm * qi[e] * ei;
          }
          const FragS fa = P::cmp8(xa), fk = P::cmp8(xk), fq = P::cmp8(xq);
#pragma unroll
          for (int t = 0; t < 3; ++t) {
            la[t] = term(fa, fk, la[t], t);
            pa[t] = term(fa, fq, pa[t], t);
          }
        }
        lacc = la[0] + la[1] + la[2];
        pacc = pa[0] + pa[1] + pa[2];
      } else {
        // pair by pair: element (i, j = 16 I + 4 g + r), channels four at a time
        for (int c4 = 0; c4 < K; c4 += 4) {
          const u32x2 qu = *reinterpret_cast<const u32x2*>(qi_row + c4);
          const f32x4 qv = {__uint_as_float(qu[0] << 16), __uint_as_float(qu[0] & 0xffff0000u),
                            __uint_as_float(qu[1] << 16), __uint_as_float(qu[1] & 0xffff0000u)};
          const u32x2 ku = *reinterpret_cast<const u32x2*>(&sK[i * LDK + c4]);
          const f32x4 kv = {__uint_as_float(ku[0] << 16), __uint_as_float(ku[0] & 0xffff0000u),
                            __uint_as_float(ku[1] << 16), __uint_as_float(ku[1] & 0xffff0000u)};
          const f32x4 gv = *reinterpret_cast<const f32x4*>(&sG[i * LDG + c4]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * I + 4 * lg + r;
            const u32x2 ju = *reinterpret_cast<const u32x2*>(&sK[j * LDK + c4]);
            const f32x4 kjv = {__uint_as_float(ju[0] << 16), __uint_as_float(ju[0] & 0xffff0000u),
                               __uint_as_float(ju[1] << 16), __uint_as_float(ju[1] & 0xffff0000u)};
            const f32x4 gjv = *reinterpret_cast<const f32x4*>(&sG[j * LDG + c4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // exponents of the pairs above the diagonal (discarded) are kept <= 0
              const float wgt = kjv[e] * exp2_hw(fminf(gv[e] - gjv[e], 0.f));
              lacc[r] = fmaf(kv[e], wgt, lacc[r]);
              pacc[r] = fmaf(qv[e], wgt, pacc[r]);
            }
          }
        }
        pacc *= qm;
      }
      f32x4 lv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * J + 4 * lg + r;
        lv[r] = j < i ? bi * lacc[r] : 0.f;
        pt[half][r] = j <= i ? pacc[r] : 0.f;
      }
      *reinterpret_cast<f32x4*>(&sLA[i][16 * J + 4 * lg]) = lv;
    }
    P::st_cmp(ops + Ops::pf + kda_a_tile(I, ks) * Ops::kFrag, lane, P::cmp_tiles(pt[0], pt[1]));
  }
  __syncthreads();

  // (2) D_w = (I + L_ww)^-1 by forward substitution (lane (j, part) keeps rows
  // [4 part, 4 part + 4) of column j; the parts are added by quad permutations),
  // then this wave's share of the state-side operands
  {
    const int j = lane >> 2, part = lane & 3;
    f32x4 lrow[15];
#pragma unroll
    for (int i = 1; i < 16; ++i) lrow[i - 1] = *reinterpret_cast<const f32x4*>(&sLA[16 * w + i][16 * w + 4 * part]);
    f32x4 av;
#pragma unroll
    for (int r = 0; r < 4; ++r) av[r] = (4 * part + r == j) ? 1.f : 0.f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      float s = (lrow[i - 1][0] * av[0] + lrow[i - 1][1] * av[1]) + (lrow[i - 1][2] * av[2] + lrow[i - 1][3] * av[3]);
      s += quad_xor1(s);
      s += quad_xor2(s);
      if (part == (i >> 2) && i > j) av[i & 3] = -s;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sLA[16 * w + 4 * part + r][16 * w + j] = av[r];
  }
  {
    // K o e^G and s q o e^G, row tile w
    const int i = 16 * w + lc;
    const float qm = i < n ? scale : 0.f;
    const __bf16* qi_row = q_row(i);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float ki[8], gi8[8], qi[8], xk[8], xq[8];
      kda_row8(sK + i * LDK, 32 * kb, lg, ki);
      kda_row8(sG + i * LDG, 32 * kb, lg, gi8);
      kda_row8(qi_row, 32 * kb, lg, qi);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float eg = exp2_hw(gi8[e]);
        xk[e] = ki[e] * eg;
        xq[e] = qm * qi[e] * eg;
      }
      P::st_cmp(ops + Ops::kg + (w * NKB + kb) * Ops::kFrag, lane, P::cmp8(xk));
      P::st_cmp(ops + Ops::qg + (w * NKB + kb) * Ops::kFrag, lane, P::cmp8(xq));
    }
    // (K o e^{G_last - G})^T, key tiles TPW w .. TPW w + TPW - 1
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = TPW * w + u, key = 16 * t + lc;
      const float gL = sG[63 * LDG + key];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jt = 32 * tb + kappa(lg, e);
          x[e] = static_cast<float>(sK[jt * LDK + key]) * exp2_hw(gL - sG[jt * LDG + key]);
        }
        P::st_cmp(ops + Ops::kdt + (2 * t + tb) * Ops::kFrag, lane, P::cmp8(x));
      }
    }
    if (tid < K) reinterpret_cast<float*>(ops + Ops::gl)[tid] = exp2_hw(sG[63 * LDG + tid]);
  }
  __syncthreads();

  // (3) the blocks below the diagonal by distance d from it,
  // A_ij = -D_i sum_{j <= m < i} L_im A_mj (waves 0 .. 3 - d)
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int jb = w, ib = w + d;
      f32x4 x = zero4();
#pragma unroll
      for (int kb = jb; kb < ib; ++kb) {
        const f32x4 lik = *reinterpret_cast<const f32x4*>(&sLA[16 * ib + lc][16 * kb + 4 * lg]);
        f32x4 akj;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          akj[e] = kb == jb ? sLA[16 * jb + 4 * lg + e][16 * jb + lc] : sOff[off_block(kb, jb)][4 * lg + e][lc];
        x = kda_mma16v(lik, akj, x);
      }
      const f32x4 di = *reinterpret_cast<const f32x4*>(&sLA[16 * ib + lc][16 * ib + 4 * lg]);
      const f32x4 y = kda_mma16v(di, x, zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) sOff[off_block(ib, jb)][4 * lg + r][lc] = -y[r];
    }
    __syncthreads();
  }

  // (4) A' = A diag(beta): wave w writes row tile w, token blocks 0 and (row
  // tiles 2, 3) 1
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (ks > 0 && w < 2) continue;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int m = 32 * ks + kappa(lg, e);
      const int mb = m >> 4;
      const float av = mb == w ? sLA[16 * w + lc][m] : mb < w ? sOff[off_block(w, mb)][lc][m & 15] : 0.f;
      x[e] = av * sB[m];
    }
    P::st_cmp(ops + Ops::af + kda_a_tile(w, ks) * Ops::kFrag, lane, P::cmp8(x));
  }
}

// One workgroup (4 waves) per (value slice of 16 columns, head, sequence). Wave
// w owns token rows 16 w .. 16 w + 15 of R, D and o, and the state's key tiles
// TPW w .. TPW w + TPW - 1 (16 keys x 16 columns each, lane (g, c) holding keys
// 16 t + 4 g + r of column c) in MFMA accumulators. Per chunk:
//   (1) R = V - (K o e^G) h, its row tile into LDS as half a B operand;
//   (2) D = A' R (row tile w), into LDS the same way;
//   (3) h <- diag(e^{G_last}) h + (K o e^{G_last - G})^T D on the wave's key
//       tiles, published as B operands for the next chunk (double buffered);
//   (4) o = (s q o e^G) h + P D from the state the chunk started with.
// The chunk's operands (about 130 KB per workgroup) are what bounds a step:
// their loads are spread over the step, each issued right after the last use
// of the registers it refills.
// Three barriers per chunk.
template <int K, typename Tout>
__global__ __launch_bounds__(256) void kda_scan_split_kernel(const __bf16* __restrict__ v,
                                                             const char* __restrict__ ws, Tout* __restrict__ o,
                                                             KdaScanArgs a) {
  using P = Prec<__bf16>;
  using Ops = KdaOps<K>;
  constexpr int NKB = K / 32, TPW = K / 64, F = Ops::kFrag;
  __shared__ __attribute__((aligned(16))) char hB[2][NKB][F];  // the state as B operands (key blocks)
  __shared__ __attribute__((aligned(16))) char rB[2][F];       // R as B operands (token blocks)
  __shared__ __attribute__((aligned(16))) char dB[2][F];       // D as B operands (token blocks)
  KdaSeq s;
  if (!kda_seq_of(a, s)) return;
  const int H = a.H, V = a.V, h = s.h;
  const int NC = (s.len + 63) / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, lc = lane & 15;
  const float* st_in;
  float* st_out;
  kda_pages<K>(a, s, st_in, st_out);
  const int64_t st_row = static_cast<int64_t>(s.v_base) * K;  // this slice's rows of the [V, K] page

  f32x4 hs[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = TPW * w + u;
    hs[u] = st_in ? *reinterpret_cast<const f32x4*>(st_in + st_row + lc * K + 16 * t + 4 * lg) : zero4();
    P::st_tile(hB[0][t >> 1], lane, t & 1, hs[u]);
  }
  const char* ops0 = ws + (static_cast<int64_t>(s.chunk0) * H + h) * Ops::bytes;
  const int64_t cstride = static_cast<int64_t>(H) * Ops::bytes;
  // Global accesses go through buffer descriptors: a chunk's fragment block
  // (uniform offsets in scalar registers, lane * 16 the only per-lane offset),
  // and the chunk's V and o rows of this head and slice, the descriptor ending
  // at the chunk's last row (rows past it read as zeros, their stores are
  // dropped).
  const uint32_t HV = static_cast<uint32_t>(H) * V;
  uint32_t row_el[4];  // element offsets of rows 16 w + 4 g + r, column c, within a chunk
#pragma unroll
  for (int r = 0; r < 4; ++r) row_el[r] = static_cast<uint32_t>(16 * w + 4 * lg + r) * HV + lc;
  auto rows_buf = [&](const void* base_el, int ch, int esize) {
    const int n = min(64, s.len - 64 * ch);
    const int64_t first = (static_cast<int64_t>(s.start) + 64 * ch) * H + h;
    return Buf(static_cast<const char*>(base_el) + (first * V + s.v_base) * esize,
               static_cast<uint32_t>(((n - 1) * HV + 16) * esize));
  };
  const uint32_t lo16 = lane * 16;

  FragS kg[NKB], qg[NKB], af[2], pf[2], kd[TPW][2];
  f32x4 gl[TPW];
  uint16_t vr[4];
  auto frag = [&](const Buf& b, int off) {
    return FragS{as_bf16x8(b.load16(lo16, off)), as_bf16x8(b.load16(lo16, off + 1024))};
  };
  auto ld_kg = [&](const Buf& b) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) kg[kb] = frag(b, Ops::kg + (w * NKB + kb) * F);
  };
  auto ld_qg = [&](const Buf& b) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) qg[kb] = frag(b, Ops::qg + (w * NKB + kb) * F);
  };
  auto ld_af = [&](const Buf& b) {
    af[0] = frag(b, Ops::af + kda_a_tile(w, 0) * F);
    if (w >= 2) af[1] = frag(b, Ops::af + kda_a_tile(w, 1) * F);
  };
  auto ld_pf = [&](const Buf& b) {
    pf[0] = frag(b, Ops::pf + kda_a_tile(w, 0) * F);
    if (w >= 2) pf[1] = frag(b, Ops::pf + kda_a_tile(w, 1) * F);
  };
  auto ld_kd = [&](const Buf& b) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = TPW * w + u;
      kd[u][0] = frag(b, Ops::kdt + (2 * t) * F);
      kd[u][1] = frag(b, Ops::kdt + (2 * t + 1) * F);
      gl[u] = __builtin_bit_cast(f32x4, b.load16(static_cast<uint32_t>(16 * t + 4 * lg) * 4, Ops::gl));
    }
  };
  auto ld_v = [&](int ch) {  // rows 16 w + 4 g + r of chunk ch, column v_base + c (0 past the end)
    const Buf vb = rows_buf(v, ch, 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) vr[r] = vb.load2(row_el[r] * 2, 0);
  };
  if (NC > 0) {
    // in the order the loop issues them: the memory counter is waited on by
    // position, and the wait at the loop head serves both ways into it
    const Buf b0(ops0, Ops::bytes);
    ld_kg(b0);
    ld_v(0);
    ld_af(b0);
    ld_kd(b0);
    ld_qg(b0);
    ld_pf(b0);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) af[i] = pf[i] = FragS{zero_bf16x8(), zero_bf16x8()};
  }
  __syncthreads();  // the initial state is published

  int cur = 0;
  for (int ch = 0; ch < NC; ++ch) {
    const Buf nx(ops0 + static_cast<int64_t>(min(ch + 1, NC - 1)) * cstride, Ops::bytes);
    float vc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) vc[r] = __uint_as_float(static_cast<uint32_t>(vr[r]) << 16);

    // (1) R = V - (K o e^G) h
    FragS hb[NKB];
    f32x4 z[3] = {zero4(), zero4(), zero4()};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      hb[kb] = P::ld_cmp(hB[cur][kb], lane);
#pragma unroll
      for (int t = 0; t < 3; ++t) z[t] = term(kg[kb], hb[kb], z[t], t);
    }
    const f32x4 zz = z[0] + z[1] + z[2];
    P::st_tile(rB[w >> 1], lane, w & 1, f32x4{vc[0] - zz[0], vc[1] - zz[1], vc[2] - zz[2], vc[3] - zz[3]});
    ld_kg(nx);
    ld_v(min(ch + 1, NC - 1));
    __syncthreads();

    // (2) D = A' R (A' vanishes above the diagonal: token block 1 only for row tiles 2, 3)
    f32x4 d[3] = {zero4(), zero4(), zero4()};
    {
      const FragS r0 = P::ld_cmp(rB[0], lane);
#pragma unroll
      for (int t = 0; t < 3; ++t) d[t] = term(af[0], r0, d[t], t);
    }
    if (w >= 2) {
      const FragS r1 = P::ld_cmp(rB[1], lane);
#pragma unroll
      for (int t = 0; t < 3; ++t) d[t] = term(af[1], r1, d[t], t);
    }
    P::st_tile(dB[w >> 1], lane, w & 1, d[0] + d[1] + d[2]);
    ld_af(nx);
    __syncthreads();

    // (3) h <- diag(e^{G_last}) h + (K o e^{G_last - G})^T D
    const FragS db[2] = {P::ld_cmp(dB[0], lane), P::ld_cmp(dB[1], lane)};
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = TPW * w + u;
      f32x4 acc[3] = {gl[u] * hs[u], zero4(), zero4()};
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int tt = 0; tt < 3; ++tt) acc[tt] = term(kd[u][tb], db[tb], acc[tt], tt);
      hs[u] = acc[0] + acc[1] + acc[2];
      P::st_tile(hB[cur ^ 1][t >> 1], lane, t & 1, hs[u]);
    }
    ld_kd(nx);

    // (4) o = (s q o e^G) h + P D, h the state the chunk started with
    f32x4 oc[3] = {zero4(), zero4(), zero4()};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 3; ++t) oc[t] = term(qg[kb], hb[kb], oc[t], t);
#pragma unroll
    for (int t = 0; t < 3; ++t) oc[t] = term(pf[0], db[0], oc[t], t);
    if (w >= 2) {
#pragma unroll
      for (int t = 0; t < 3; ++t) oc[t] = term(pf[1], db[1], oc[t], t);
    }
    const f32x4 ov = oc[0] + oc[1] + oc[2];
    {
      const Buf ob = rows_buf(o, ch, sizeof(Tout));
#pragma unroll
      for (int r = 0; r < 4; ++r) ob.store(static_cast<Tout>(ov[r]), row_el[r] * sizeof(Tout), 0);
    }
    ld_qg(nx);
    ld_pf(nx);
    cur ^= 1;
    __syncthreads();  // the new state is published; every wave is done with R, D and the old state
  }
  if (st_out) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = TPW * w + u;
      *reinterpret_cast<f32x4*>(st_out + st_row + lc * K + 16 * t + 4 * lg) = hs[u];
    }
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
  const KdaChunkGeo geo{varlen ? info : nullptr, a.T_eq, ncs_eq, static_cast<int>(a.total_tokens)};
  constexpr bool kSplit = std::is_same<Tin, __bf16>::value;
  if (a.n_chunks > 0) {
    if constexpr (kSplit)
      hipLaunchKernelGGL((kda_prep_split_kernel<K>), dim3(static_cast<unsigned>(a.n_chunks), a.H), dim3(256), 0,
                         a.stream, static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k), a.g, a.beta,
                         static_cast<char*>(a.ws), geo, a.H, a.scale);
    else
      hipLaunchKernelGGL((kda_prep_kernel<K, Tin>), dim3(static_cast<unsigned>(a.n_chunks), a.H), dim3(kPrepThreads),
                         0, a.stream, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), a.g, a.beta, ops, geo,
                         a.H, a.scale);
  }
  if (a.events[1]) (void)hipEventRecord(a.events[1], a.stream);
  KdaScanArgs sa{a.h0, a.ht, a.pool, a.pool_slots, a.slots, a.H, a.V, a.n_seqs, a.T_eq, ncs_eq,
                 static_cast<int>(a.total_tokens), static_cast<int>(a.n_chunks), a.cu_seqlens, seq_chunk0};
  const int64_t n_pairs = static_cast<int64_t>(a.n_seqs) * a.H;
  const dim3 grid(static_cast<unsigned>((n_pairs + 7) / 8) * 8 * (a.V / kKdaSlice));
  if constexpr (kSplit) {
    if (a.out_f32)
      hipLaunchKernelGGL((kda_scan_split_kernel<K, float>), grid, dim3(256), 0, a.stream,
                         static_cast<const __bf16*>(a.v), static_cast<const char*>(a.ws), static_cast<float*>(a.o), sa);
    else
      hipLaunchKernelGGL((kda_scan_split_kernel<K, __bf16>), grid, dim3(256), 0, a.stream,
                         static_cast<const __bf16*>(a.v), static_cast<const char*>(a.ws), static_cast<__bf16*>(a.o),
                         sa);
    return;
  }
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

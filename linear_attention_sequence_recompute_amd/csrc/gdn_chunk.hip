// Chunked forward pass of the gated delta rule on gfx950.
//
// The WarpDrive page chains three kernels over chunks of C = 64 tokens:
// recompute_w_u (u = A (v beta), w = A (k beta e^g) with the chunk's WY matrix A),
// chunk_fwd_h (the sequential state recurrence over a [K, V] state) and
// chunk_fwd_o (inter-chunk q h e^g plus the causally masked intra-chunk term).
// This file runs them as two launches (plus a schedule launch for packed
// sequences):
//
//  * prep_kernel, one workgroup per (chunk, head), fully parallel: the
//    chunk-local gate cumsum, K K^T -> L, the triangular solve A = (I + L)^-1 in
//    LDS, u and w, the masked score matrix P of chunk_fwd_o and K^T, all written
//    in the MFMA operand order the scan kernel reads.
//  * scan_kernel, one workgroup per (sequence, head, slice of V): the sequential
//    chunk loop of chunk_fwd_h with chunk_fwd_o fused into it, so the per-chunk
//    states and v_new never leave the chip. The state slice lives in MFMA
//    accumulator registers for the whole sequence; each wave owns 32 key rows of
//    it, the decay e^{g_last} is folded into the accumulator before K^T v_gated
//    is added, and the partial products over key rows are summed through LDS.
//
// Precision: q, k, v are exact in bf16 and enter the MFMA as one operand; every
// computed operand (A diag(beta), A diag(beta e^g), w, h, v_new, P) enters as a
// bf16 hi + lo pair with fp32 accumulation, which keeps about 16 significant bits.
// Float32 inputs are split the same way.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kLdt = 68;  // padded row length (elements) of the transposed LDS tiles

__device__ __forceinline__ bf16x8 ld_frag(const __bf16* p) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_frag(__bf16* p, bf16x8 x) {
  *reinterpret_cast<u32x4*>(p) = as_u32x4(x);
}

// Reads the kappa-ordered 8 elements of row `row` of a transposed LDS tile,
// contraction block starting at column c0.
__device__ __forceinline__ bf16x8 lds_frag(const __bf16* tile, int row, int c0, int g) {
  const __bf16* p = tile + row * kLdt + c0;
  u32x2 a = *reinterpret_cast<const u32x2*>(p + 4 * g);
  u32x2 b = *reinterpret_cast<const u32x2*>(p + 16 + 4 * g);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

// ---------------------------------------------------------------------------
// Chunk schedule of a packed call: chunk c of sequence s gets global index
// seq_chunk0[s] + c and its {seq, first token, rows} entry. One workgroup.
// ---------------------------------------------------------------------------
// Entries past the schedule are marked empty, and a sequence whose offsets do
// not fit [0, total_tokens] or whose chunks would pass `cap` gets none, so an
// inconsistent device copy of the offsets cannot steer any access out of bounds.
__global__ __launch_bounds__(256) void schedule_kernel(const int32_t* __restrict__ cu, int n_seqs,
                                                       int total_tokens, int cap,
                                                       int* __restrict__ seq_chunk0,
                                                       int4* __restrict__ info) {
  __shared__ int wsum[4];
  __shared__ int carry;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < cap; i += 256) info[i] = int4{-1, 0, 0, 0};
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n_seqs; base += 256) {
    const int s = base + tid;
    int start = 0, len = 0;
    if (s < n_seqs) {
      start = cu[s];
      len = cu[s + 1] - start;
      if (start < 0 || len < 0 || start > total_tokens - len) len = 0;
    }
    const int nc = (len + kChunk - 1) / kChunk;
    int incl = nc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int before = carry;
    for (int i = 0; i < w; ++i) before += wsum[i];
    const int first = before + incl - nc;
    if (s < n_seqs) {
      seq_chunk0[s] = first;
      for (int c = 0; c < nc && first + c < cap; ++c)
        info[first + c] = int4{s, start + kChunk * c, min(kChunk, len - kChunk * c), 0};
    }
    __syncthreads();
    if (tid == 255) carry = first + nc;
    __syncthreads();
  }
  if (tid == 0) seq_chunk0[n_seqs] = carry;
}

// ---------------------------------------------------------------------------
// recompute_w_u (+ the pieces of chunk_fwd_o that do not depend on the state).
// ---------------------------------------------------------------------------
template <int K, int V, typename Tin>
__global__ __launch_bounds__(256) void prep_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                                                   const Tin* __restrict__ v, const float* __restrict__ g,
                                                   const float* __restrict__ beta, int H, float scale,
                                                   int T_eq, int ncs_eq, int total_tokens,
                                                   const int4* __restrict__ info, ChunkWs ws) {
  constexpr int NP = In<Tin>::kParts;
  __shared__ __attribute__((aligned(16))) __bf16 sKt[NP][K][kLdt];  // K^T: [key][token]
  __shared__ __attribute__((aligned(16))) __bf16 sVt[NP][V][kLdt];  // V^T: [value][token]
  __shared__ float sL[64][65];
  __shared__ float sA[64][65];
  __shared__ float sg[64], sb[64], sbeg[64];

  const int c = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;
  int t0, n;
  if (info) {
    const int4 ci = info[c];
    t0 = ci.y;
    n = ci.z;
    if (ci.x < 0 || n <= 0 || n > kChunk || t0 < 0 || t0 > total_tokens - n) return;
  } else {
    const int s = c / ncs_eq, j = c % ncs_eq;
    t0 = s * T_eq + kChunk * j;
    n = min(kChunk, T_eq - kChunk * j);
  }
  const int64_t ch = static_cast<int64_t>(c) * H + h;

  // (1) chunk-local inclusive cumsum of the log-gate; beta; beta e^g.
  if (w == 0) {
    const int64_t gi = static_cast<int64_t>(t0 + lane) * H + h;
    const float a = lane < n ? g[gi] : 0.f;
    const float gl = wave_inclusive_scan(a);
    const float bl = lane < n ? beta[gi] : 0.f;
    sg[lane] = gl;
    sb[lane] = bl;
    sbeg[lane] = bl * __expf(gl);
    ws.gc[ch * kChunk + lane] = gl;
  }
  // (2) transposed copies of the chunk's K and V (rows past the end are zero).
  {
    const int per_row = K / 8;
    for (int id = tid; id < kChunk * per_row; id += 256) {
      const int t = id / per_row, c8 = (id % per_row) * 8;
      float x[8];
      if (t < n) {
        const Tin* p = k + (static_cast<int64_t>(t0 + t) * H + h) * K + c8;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = In<Tin>::ld(p + e);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 hi, lo;
        split1(x[e], hi, lo);
        sKt[0][c8 + e][t] = hi;
        if constexpr (NP == 2) sKt[NP - 1][c8 + e][t] = lo;
      }
    }
  }
  {
    const int per_row = V / 8;
    for (int id = tid; id < kChunk * per_row; id += 256) {
      const int t = id / per_row, c8 = (id % per_row) * 8;
      float x[8];
      if (t < n) {
        const Tin* p = v + (static_cast<int64_t>(t0 + t) * H + h) * V + c8;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = In<Tin>::ld(p + e);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 hi, lo;
        split1(x[e], hi, lo);
        sVt[0][c8 + e][t] = hi;
        if constexpr (NP == 2) sVt[NP - 1][c8 + e][t] = lo;
      }
    }
  }
  // identity init of A
  for (int idx = tid; idx < 64 * 64; idx += 256) sA[idx >> 6][idx & 63] = (idx >> 6) == (idx & 63) ? 1.f : 0.f;
  __syncthreads();

  auto krow_frag = [&](const Tin* base, int D, int row, int kb, bf16x8& hi, bf16x8& lo) {
    if (row < n) {
      In<Tin>::row_frag(base + (static_cast<int64_t>(t0 + row) * H + h) * D + 32 * kb, lg, hi, lo);
    } else {
      hi = zero_bf16x8();
      lo = zero_bf16x8();
    }
  };

  // (3) L = StrictLower(diag(beta) K K^T * E): the 10 lower 16x16 tiles.
  for (int tix = w; tix < 10; tix += 4) {
    const int bi = tix == 0 ? 0 : tix < 3 ? 1 : tix < 6 ? 2 : 3;
    const int bj = tix - (bi * (bi + 1)) / 2;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
      bf16x8 ahi, alo, bhi, blo;
      krow_frag(k, K, 16 * bi + lc, kb, ahi, alo);
      krow_frag(k, K, 16 * bj + lc, kb, bhi, blo);
      acc = mma_split<NP, NP>(ahi, alo, bhi, blo, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * bi + 4 * lg + r, j = 16 * bj + lc;
      sL[i][j] = j < i ? sb[i] * acc[r] * __expf(sg[i] - sg[j]) : 0.f;
    }
  }

  // (4) P = s (Q K^T) * E * M, computed transposed so that accumulator tiles are
  // directly the A operands of P: wave w owns output row tile w.
  {
    const int bi = w;
    const int nks = bi >= 2 ? 2 : 1;
    for (int ks = 0; ks < 2; ++ks) {
      f32x4 d[2] = {zero4(), zero4()};
      if (ks < nks) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int bt = 2 * ks + half;
          if (bt > bi) continue;
#pragma unroll
          for (int kb = 0; kb < K / 32; ++kb) {
            bf16x8 ahi, alo, bhi, blo;
            krow_frag(k, K, 16 * bt + lc, kb, ahi, alo);
            krow_frag(q, K, 16 * bi + lc, kb, bhi, blo);
            d[half] = mma_split<NP, NP>(ahi, alo, bhi, blo, d[half]);
          }
          const int i = 16 * bi + lc;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tp = 16 * bt + 4 * lg + r;
            d[half][r] = tp <= i ? scale * d[half][r] * __expf(sg[i] - sg[tp]) : 0.f;
          }
        }
      }
      bf16x8 phi, plo;
      split_tiles(d[0], d[1], phi, plo);
      __bf16* dst = ws.pf + ch * 8192 + ((bi * 2 + ks) * 2) * 512 + lane * 8;
      st_frag(dst, phi);
      st_frag(dst + 512, plo);
    }
  }
  __syncthreads();

  // (5) A = (I + L)^-1 by forward substitution, one row per step: thread
  // (j, part) sums a quarter of row i's terms for column j.
  {
    const int j = tid >> 2, part = tid & 3;
    for (int i = 1; i < 64; ++i) {
      float s = 0.f;
      if (j < i)
        for (int m = j + part; m < i; m += 4) s += sL[i][m] * sA[m][j];
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      if (part == 0 && j < i) sA[i][j] = -s;
      __syncthreads();
    }
  }

  // (6) u = A diag(beta) V, wave w owns output row tile w (all value tiles).
  {
    constexpr int NVT = V / 16;
    f32x4 acc[NVT];
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) acc[vt] = zero4();
    const int nks = w >= 2 ? 2 : 1;
    for (int ks = 0; ks < nks; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = 32 * ks + kappa(lg, e);
        x[e] = sA[16 * w + lc][m] * sb[m];
      }
      bf16x8 ahi, alo;
      split8(x, ahi, alo);
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const bf16x8 bhi = lds_frag(&sVt[0][0][0], 16 * vt + lc, 32 * ks, lg);
        const bf16x8 blo = NP == 2 ? lds_frag(&sVt[NP - 1][0][0], 16 * vt + lc, 32 * ks, lg) : zero_bf16x8();
        acc[vt] = mma_split<2, NP>(ahi, alo, bhi, blo, acc[vt]);
      }
    }
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt)
      *reinterpret_cast<f32x4*>(ws.uf + ch * (V * 64) + ((vt * 4 + w) * 64 + lane) * 4) = acc[vt];
  }

  // (7) w = A diag(beta e^g) K, computed as w^T = K^T (A diag(beta e^g))^T so that
  // pairs of accumulator tiles are the A operands of w over a 32-key block.
  {
    constexpr int NKT = K / 16;
    f32x4 acc[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) acc[kt] = zero4();
    const int nks = w >= 2 ? 2 : 1;
    for (int ks = 0; ks < nks; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = 32 * ks + kappa(lg, e);
        x[e] = sA[16 * w + lc][m] * sbeg[m];
      }
      bf16x8 bhi, blo;
      split8(x, bhi, blo);
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const bf16x8 ahi = lds_frag(&sKt[0][0][0], 16 * kt + lc, 32 * ks, lg);
        const bf16x8 alo = NP == 2 ? lds_frag(&sKt[NP - 1][0][0], 16 * kt + lc, 32 * ks, lg) : zero_bf16x8();
        acc[kt] = mma_split<NP, 2>(ahi, alo, bhi, blo, acc[kt]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
      bf16x8 hi, lo;
      split_tiles(acc[2 * kb], acc[2 * kb + 1], hi, lo);
      __bf16* dst = ws.wf + ch * (K * 128) + ((kb * 4 + w) * 2) * 512 + lane * 8;
      st_frag(dst, hi);
      st_frag(dst + 512, lo);
    }
  }

  // (8) K^T as A operands for the state update of the scan kernel.
  for (int idx = w; idx < (K / 16) * 2; idx += 4) {
    const int kt = idx >> 1, ks = idx & 1;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const bf16x8 f = lds_frag(&sKt[p][0][0], 16 * kt + lc, 32 * ks, lg);
      st_frag(ws.ktf + ch * (K * 64 * NP) + ((kt * 2 + ks) * NP + p) * 512 + lane * 8, f);
    }
  }
}

// ---------------------------------------------------------------------------
// chunk_fwd_h with chunk_fwd_o fused: sequential over the chunks of one
// sequence, for one head and one slice of 16 * NSUB value columns.
// ---------------------------------------------------------------------------
template <int K, int V, int NSUB, typename Tin, typename Tout>
__global__ __launch_bounds__(K / 32 * 64) void scan_kernel(
    const Tin* __restrict__ q, Tout* __restrict__ o, int H, float scale, int n_seqs, int T_eq,
    int ncs_eq, int total_tokens, int n_chunks, const int32_t* __restrict__ cu, const float* __restrict__ h0, float* __restrict__ ht,
    float* __restrict__ pool, int64_t pool_slots, const int32_t* __restrict__ slots, ChunkWs ws) {
  constexpr int NW = K / 32;          // waves; wave w owns key rows [32w, 32w + 32)
  constexpr int NP = In<Tin>::kParts;
  constexpr int RT = 4 / NW;          // output row tiles each wave finishes
  constexpr int NSL = V / (16 * NSUB);
  __shared__ f32x4 sX[NW][4][NSUB][64];  // partial w h over this wave's key rows
  __shared__ f32x4 sY[NW][4][NSUB][64];  // partial q h
  __shared__ u32x2 sVn[4][NSUB][4][64];  // v_new hi, lo and gated v_new hi, lo (4 bf16 each)

  // Workgroups of one (sequence, head) share an XCD (blockIdx % 8) and its L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, rest = bid >> 3;
  const int slice = rest % NSL;
  const int pair = (rest / NSL) * 8 + xcd;
  if (pair >= n_seqs * H) return;
  const int seq = pair / H, h = pair % H;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;
  int start, len, chunk0;
  if (cu) {
    start = cu[seq];
    len = cu[seq + 1] - start;
    chunk0 = ws.seq_chunk0[seq];
    const int nc_want = (len + kChunk - 1) / kChunk;
    if (start < 0 || len < 0 || start > total_tokens - len || chunk0 < 0 || chunk0 > n_chunks - nc_want) len = 0;
  } else {
    start = seq * T_eq;
    len = T_eq;
    chunk0 = seq * ncs_eq;
  }
  const int nc = (len + kChunk - 1) / kChunk;

  const float* s_in = nullptr;
  float* s_out = nullptr;
  const int64_t page = static_cast<int64_t>(V) * K;
  if (pool) {
    const int s = slots[seq];
    if (s > 0 && s < pool_slots) {
      s_in = pool + (static_cast<int64_t>(s) * H + h) * page;
      s_out = pool + (static_cast<int64_t>(s) * H + h) * page;
    }
  } else {
    if (h0) s_in = h0 + (static_cast<int64_t>(seq) * H + h) * page;
    if (ht) s_out = ht + (static_cast<int64_t>(seq) * H + h) * page;
  }

  // State slice h[key][value] = S[value][key]: two accumulator tiles per 16 columns.
  f32x4 hs[NSUB][2];
#pragma unroll
  for (int ns = 0; ns < NSUB; ++ns) {
    const int vcol = (slice * NSUB + ns) * 16 + lc;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int k0 = 32 * w + 16 * tt + 4 * lg;
      hs[ns][tt] = s_in ? *reinterpret_cast<const f32x4*>(s_in + static_cast<int64_t>(vcol) * K + k0) : zero4();
    }
  }

  for (int c = 0; c < nc; ++c) {
    const int64_t ch = static_cast<int64_t>(chunk0 + c) * H + h;
    const int t0 = start + kChunk * c;
    const int n = min(kChunk, len - kChunk * c);
    const float* gch = ws.gc + ch * kChunk;
    const float gL = gch[kChunk - 1];

    // (1) the state as hi/lo B operands of this wave's 32-key block
    bf16x8 hhi[NSUB], hlo[NSUB];
#pragma unroll
    for (int ns = 0; ns < NSUB; ++ns) split_tiles(hs[ns][0], hs[ns][1], hhi[ns], hlo[ns]);

    // (2) partial w h and q h over this wave's key rows, all 64 chunk rows
    const __bf16* wf = ws.wf + ch * (K * 128) + (w * 4 * 2) * 512 + lane * 8;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const bf16x8 whi = ld_frag(wf + (rt * 2) * 512);
      const bf16x8 wlo = ld_frag(wf + (rt * 2 + 1) * 512);
      bf16x8 qhi, qlo;
      const int row = 16 * rt + lc;
      if (row < n) {
        In<Tin>::row_frag(q + (static_cast<int64_t>(t0 + row) * H + h) * K + 32 * w, lg, qhi, qlo);
      } else {
        qhi = zero_bf16x8();
        qlo = zero_bf16x8();
      }
#pragma unroll
      for (int ns = 0; ns < NSUB; ++ns) {
        sX[w][rt][ns][lane] = mma_split<2, 2>(whi, wlo, hhi[ns], hlo[ns], zero4());
        sY[w][rt][ns][lane] = mma_split<NP, 2>(qhi, qlo, hhi[ns], hlo[ns], zero4());
      }
    }
    __syncthreads();

    // (3) this wave's output row tiles: v_new = u - w h, gated v_new, inter part
    f32x4 acc_o[RT][NSUB];
#pragma unroll
    for (int rho = 0; rho < RT; ++rho) {
      const int rt = w * RT + rho;
      float gr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) gr[r] = gch[16 * rt + 4 * lg + r];
#pragma unroll
      for (int ns = 0; ns < NSUB; ++ns) {
        f32x4 x = sX[0][rt][ns][lane], y = sY[0][rt][ns][lane];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) {
          x += sX[ww][rt][ns][lane];
          y += sY[ww][rt][ns][lane];
        }
        const f32x4 u =
            *reinterpret_cast<const f32x4*>(ws.uf + ch * (V * 64) + (((slice * NSUB + ns) * 4 + rt) * 64 + lane) * 4);
        bf16x4 vnh, vnl, vgh, vgl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float vn = u[r] - x[r];
          const float vg = vn * __expf(gL - gr[r]);
          acc_o[rho][ns][r] = scale * __expf(gr[r]) * y[r];
          __bf16 a, b;
          split1(vn, a, b);
          vnh[r] = a;
          vnl[r] = b;
          split1(vg, a, b);
          vgh[r] = a;
          vgl[r] = b;
        }
        sVn[rt][ns][0][lane] = __builtin_bit_cast(u32x2, vnh);
        sVn[rt][ns][1][lane] = __builtin_bit_cast(u32x2, vnl);
        sVn[rt][ns][2][lane] = __builtin_bit_cast(u32x2, vgh);
        sVn[rt][ns][3][lane] = __builtin_bit_cast(u32x2, vgl);
      }
    }
    __syncthreads();

    auto vfrag = [&](int ks, int ns, int part) {
      const u32x2 a = sVn[2 * ks][ns][part][lane];
      const u32x2 b = sVn[2 * ks + 1][ns][part][lane];
      return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
    };

    // (4) state update: h <- e^{g_last} h + K^T v_gated, decay folded into the
    // accumulator before the products are added.
    const float dL = __expf(gL);
    const __bf16* ktf = ws.ktf + ch * (K * 64 * NP) + lane * 8;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int kt = 2 * w + tt;
      bf16x8 khi[2], klo[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        khi[ks] = ld_frag(ktf + ((kt * 2 + ks) * NP) * 512);
        klo[ks] = NP == 2 ? ld_frag(ktf + ((kt * 2 + ks) * NP + NP - 1) * 512) : zero_bf16x8();
      }
#pragma unroll
      for (int ns = 0; ns < NSUB; ++ns) {
        f32x4 acc = hs[ns][tt] * dL;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc = mma_split<NP, 2>(khi[ks], klo[ks], vfrag(ks, ns, 2), vfrag(ks, ns, 3), acc);
        hs[ns][tt] = acc;
      }
    }

    // (5) o = inter + P v_new for this wave's row tiles
#pragma unroll
    for (int rho = 0; rho < RT; ++rho) {
      const int rt = w * RT + rho;
      const __bf16* pf = ws.pf + ch * 8192 + (rt * 2 * 2) * 512 + lane * 8;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks == 1 && rt < 2) continue;  // P is causal: columns >= 32 vanish for rows < 32
        const bf16x8 phi = ld_frag(pf + (ks * 2) * 512);
        const bf16x8 plo = ld_frag(pf + (ks * 2 + 1) * 512);
#pragma unroll
        for (int ns = 0; ns < NSUB; ++ns)
          acc_o[rho][ns] = mma_split<2, 2>(phi, plo, vfrag(ks, ns, 0), vfrag(ks, ns, 1), acc_o[rho][ns]);
      }
#pragma unroll
      for (int ns = 0; ns < NSUB; ++ns) {
        const int vcol = (slice * NSUB + ns) * 16 + lc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rt + 4 * lg + r;
          if (row < n) store_out(o + (static_cast<int64_t>(t0 + row) * H + h) * V + vcol, acc_o[rho][ns][r]);
        }
      }
    }
  }

  if (s_out) {
#pragma unroll
    for (int ns = 0; ns < NSUB; ++ns) {
      const int vcol = (slice * NSUB + ns) * 16 + lc;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int k0 = 32 * w + 16 * tt + 4 * lg;
        *reinterpret_cast<f32x4*>(s_out + static_cast<int64_t>(vcol) * K + k0) = hs[ns][tt];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: workspace layout and launch sequence.
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

WsLayout workspace_layout(int64_t max_chunks, int n_seqs, int H, int K, int V, bool in_f32) {
  const size_t nch = static_cast<size_t>(max_chunks) * H;
  const size_t np = in_f32 ? 2 : 1;
  WsLayout l{};
  size_t off = 0;
  l.wf = off;
  off = align256(off + nch * K * 128 * 2);
  l.ktf = off;
  off = align256(off + nch * K * 64 * np * 2);
  l.uf = off;
  off = align256(off + nch * V * 64 * 4);
  l.pf = off;
  off = align256(off + nch * 8192 * 2);
  l.gc = off;
  off = align256(off + nch * kChunk * 4);
  l.info = off;
  off = align256(off + static_cast<size_t>(max_chunks) * 16);
  l.seq_chunk0 = off;
  off = align256(off + static_cast<size_t>(n_seqs + 1) * 4);
  l.total = off;
  return l;
}

ChunkWs carve_workspace(const WsLayout& l, void* base) {
  char* b = static_cast<char*>(base);
  ChunkWs ws;
  ws.wf = reinterpret_cast<__bf16*>(b + l.wf);
  ws.ktf = reinterpret_cast<__bf16*>(b + l.ktf);
  ws.uf = reinterpret_cast<float*>(b + l.uf);
  ws.pf = reinterpret_cast<__bf16*>(b + l.pf);
  ws.gc = reinterpret_cast<float*>(b + l.gc);
  ws.info = reinterpret_cast<int4*>(b + l.info);
  ws.seq_chunk0 = reinterpret_cast<int*>(b + l.seq_chunk0);
  return ws;
}

template <int K, int V, typename Tin, typename Tout>
static hipError_t launch_chunk_t(const ChunkArgs& a) {
  constexpr int NSUB = 1;
  constexpr int NSL = V / (16 * NSUB);
  const bool varlen = a.cu_seqlens != nullptr;
  const int ncs_eq = varlen ? 0 : (a.T_eq + kChunk - 1) / kChunk;
  if (varlen) {
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(256), 0, a.stream, a.cu_seqlens, a.n_seqs,
                       static_cast<int>(a.total_tokens), static_cast<int>(a.n_chunks), a.ws.seq_chunk0,
                       a.ws.info);
  }
  if (a.n_chunks > 0) {
    hipLaunchKernelGGL((prep_kernel<K, V, Tin>), dim3(static_cast<unsigned>(a.n_chunks), a.H), dim3(256), 0,
                       a.stream, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                       static_cast<const Tin*>(a.v), a.g, a.beta, a.H, a.scale, a.T_eq, ncs_eq,
                       static_cast<int>(a.total_tokens), varlen ? a.ws.info : nullptr, a.ws);
  }
  const int64_t pairs = static_cast<int64_t>(a.n_seqs) * a.H;
  const int64_t blocks = 8 * NSL * ((pairs + 7) / 8);
  hipLaunchKernelGGL((scan_kernel<K, V, NSUB, Tin, Tout>), dim3(static_cast<unsigned>(blocks)), dim3(K / 32 * 64),
                     0, a.stream, static_cast<const Tin*>(a.q), static_cast<Tout*>(a.o), a.H, a.scale, a.n_seqs,
                     a.T_eq, ncs_eq, static_cast<int>(a.total_tokens), static_cast<int>(a.n_chunks), a.cu_seqlens, a.h0, a.ht, a.pool, a.pool_slots, a.slots, a.ws);
  return hipGetLastError();
}

template <int K, int V>
static hipError_t launch_chunk_kv(const ChunkArgs& a) {
  if (a.in_f32) return a.out_f32 ? launch_chunk_t<K, V, float, float>(a) : launch_chunk_t<K, V, float, __bf16>(a);
  return a.out_f32 ? launch_chunk_t<K, V, __bf16, float>(a) : launch_chunk_t<K, V, __bf16, __bf16>(a);
}

hipError_t launch_chunk_fwd(const ChunkArgs& a) {
  if (a.K == 128 && a.V == 128) return launch_chunk_kv<128, 128>(a);
  if (a.K == 128 && a.V == 64) return launch_chunk_kv<128, 64>(a);
  if (a.K == 64 && a.V == 128) return launch_chunk_kv<64, 128>(a);
  return launch_chunk_kv<64, 64>(a);
}

}  // namespace gdn

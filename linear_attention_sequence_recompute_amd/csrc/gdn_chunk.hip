// Chunked forward pass of the gated delta rule on gfx950.
//
// The WarpDrive page chains three kernels over chunks of C = 64 tokens:
// recompute_w_u (u = A (v beta), w = A (k beta e^g) with the chunk's WY matrix A),
// chunk_fwd_h (the sequential state recurrence over a [K, V] state) and
// chunk_fwd_o (inter-chunk q h e^g plus the causally masked intra-chunk term).
// Since u - w h = A diag(beta) (V - diag(e^g) K h), the whole chunk step only
// needs the chunk's inputs, its gate sums and A' = A diag(beta). This file runs:
//
//  * prep_kernel, one workgroup per (chunk, head), fully parallel: the
//    chunk-local gate cumsum, K K^T -> L, the triangular solve A = (I + L)^-1 in
//    LDS, and A' stored in the MFMA operand order the scan kernel reads;
//  * scan_kernel, one workgroup per (sequence, head, 16-column slice of V): the
//    sequential chunk loop of chunk_fwd_h with chunk_fwd_o fused into it. Each
//    chunk's K is staged once in LDS and serves K h, K^T (read transposed) and the
//    score matrix P = s (Q K^T) * E * M; v_new = A' (V - e^g (K h)); the state
//    lives in MFMA accumulators, the decay e^{g_last} folded into the accumulator
//    before K^T v_gated is added. Per-chunk states and v_new never leave the chip.
//
// Precision: q, k, v are exact in bf16 and enter the MFMA as one operand; every
// computed operand (A', K h residuals, h, v_new, P) enters as a bf16 hi + lo pair
// with fp32 accumulation, which keeps about 16 significant bits. Float32 inputs
// run the same code on the fp32 MFMA.
#include <type_traits>

#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kPlane = 1024;  // bytes of one fragment plane (64 lanes x 16 bytes)

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
// recompute_w_u, reduced to what the fused scan needs: the chunk-local gate
// sums and A' = A diag(beta), A = (I + StrictLower(diag(beta) K K^T * E))^-1,
// plus the state-independent score matrix P of chunk_fwd_o.
// One workgroup (4 waves) per (chunk, head).
// ---------------------------------------------------------------------------
template <int K, typename Tin>
__global__ __launch_bounds__(256) void prep_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                                                   const float* __restrict__ g, const float* __restrict__ beta,
                                                   int H, float scale, int T_eq, int ncs_eq, int total_tokens,
                                                   const int4* __restrict__ info, ChunkWs ws) {
  using P = Prec<Tin>;
  using In = typename P::In;
  constexpr int LDA = 68;  // row stride (floats) of the L / A tile: 16-byte aligned rows
  __shared__ __attribute__((aligned(16))) float sLA[64][LDA];  // L, then A
  __shared__ float sg[64], sb[64];

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

  // Row fragments of the chunk's K (rows past the end are zero).
  In kf[4][K / 32];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int row = 16 * b + lc;
    const int rowc = min(row, n - 1);
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
      kf[b][kb] = P::in_row(k + (static_cast<int64_t>(t0 + rowc) * H + h) * K + 32 * kb, lg);
      if (row >= n) kf[b][kb] = P::in_zero();
    }
  }

  // Row fragments of this wave's 16 rows of Q.
  In qf[K / 32];
  {
    const int row = 16 * w + lc;
    const int rowc = min(row, n - 1);
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
      qf[kb] = P::in_row(q + (static_cast<int64_t>(t0 + rowc) * H + h) * K + 32 * kb, lg);
      if (row >= n) qf[kb] = P::in_zero();
    }
  }

  // (1) chunk-local inclusive cumsum of the log-gate; beta; the gate vectors g,
  // e^g and e^{g_last - g} the scan kernel applies.
  if (w == 0) {
    const int64_t gi = static_cast<int64_t>(t0 + lane) * H + h;
    const float a = lane < n ? g[gi] : 0.f;
    const float gl = wave_inclusive_scan(a);
    const float glast = __shfl(gl, 63, 64);
    sg[lane] = gl;
    sb[lane] = lane < n ? beta[gi] : 0.f;
    ws.gx[ch * 192 + lane] = gl;
    ws.gx[ch * 192 + 64 + lane] = __expf(gl);
    ws.gx[ch * 192 + 128 + lane] = __expf(glast - gl);
  }
  for (int idx = tid; idx < 64 * LDA; idx += 256) (&sLA[0][0])[idx] = 0.f;
  __syncthreads();

  // (2) L = StrictLower(diag(beta) K K^T * E): the 10 lower 16x16 tiles.
#pragma unroll
  for (int tix = 0; tix < 10; ++tix) {
    if ((tix & 3) != w) continue;
    const int bi = tix == 0 ? 0 : tix < 3 ? 1 : tix < 6 ? 2 : 3;
    const int bj = tix - (bi * (bi + 1)) / 2;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) acc = mma(kf[bi][kb], kf[bj][kb], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * bi + 4 * lg + r, j = 16 * bj + lc;
      if (j < i) sLA[i][j] = sb[i] * acc[r] * __expf(sg[i] - sg[j]);
    }
  }

  // (2b) the score matrix of chunk_fwd_o, P = s (Q K^T) * E * M (E_ij = e^{g_i - g_j},
  // M the inclusive causal mask), computed transposed (P^T = K Q^T) so that pairs
  // of accumulator tiles are directly its A operands; wave w owns row tile w.
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    f32x4 d[2] = {zero4(), zero4()};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int bt = 2 * ks + half;
      if (bt > w) continue;
      f32x4 part[K / 32];
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) part[kb] = mma(kf[bt][kb], qf[kb], zero4());
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) d[half] += part[kb];
      const int i = 16 * w + lc;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tp = 16 * bt + 4 * lg + r;
        d[half][r] = tp <= i ? scale * d[half][r] * __expf(sg[i] - sg[tp]) : 0.f;
      }
    }
    P::st_cmp(ws.pf + ch * (8 * 2 * kPlane) + (w * 2 + ks) * 2 * kPlane, lane, P::cmp_tiles(d[0], d[1]));
  }
  __syncthreads();

  // (3) A = (I + L)^-1 by forward substitution without barriers: the four lanes
  // (j, part) of column j are adjacent in one wave; lane part keeps rows
  // [16 part, 16 part + 16) of column j in registers. Row i of (I + L) A = I gives
  // A[i][j] = -sum_m L[i][m] A[m][j]; each lane sums its 16 rows (L[i][m] = 0 for
  // m >= i, and A[m][j] not yet known is 0) and the four parts are added with
  // shuffles.
  {
    const int j = tid >> 2, part = tid & 3;
    float a[16];
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) a[kk] = (16 * part + kk == j) ? 1.f : 0.f;
#pragma unroll
    for (int i = 1; i < 64; ++i) {
      const f32x4* row = reinterpret_cast<const f32x4*>(&sLA[i][16 * part]);
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f32x4 l4 = row[qq];
        s0 = fmaf(l4[0], a[4 * qq + 0], s0);
        s1 = fmaf(l4[1], a[4 * qq + 1], s1);
        s2 = fmaf(l4[2], a[4 * qq + 2], s2);
        s3 = fmaf(l4[3], a[4 * qq + 3], s3);
      }
      float s = (s0 + s1) + (s2 + s3);
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      if (part == (i >> 4) && i > j) a[i & 15] = -s;
    }
    __syncthreads();  // every lane is done reading L
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) sLA[16 * part + kk][j] = a[kk];
  }
  __syncthreads();

  // (4) A' = A diag(beta) as A operands: wave w stores row tile w, token blocks
  // 0 and 1 (A' is lower triangular: block 1 of row tiles 0 and 1 is zero).
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int m = 32 * ks + kappa(lg, e);
      x[e] = sLA[16 * w + lc][m] * sb[m];
    }
    P::st_cmp(ws.af + ch * (8 * 2 * kPlane) + (w * 2 + ks) * 2 * kPlane, lane, P::cmp8(x));
  }
}

// ---------------------------------------------------------------------------
// chunk_fwd_h with chunk_fwd_o fused: sequential over the chunks of one
// sequence, for one head and one slice of 16 value columns.
//
// 2 K/32 waves in two roles meet at three barriers per chunk:
//  * chain wave w (w < K/32) owns key rows [32w, 32w + 32) of the state slice as
//    two accumulator tiles, and output row tiles [w RT, (w+1) RT). It publishes
//    its state block (barrier 1), forms Z = K h for its row tiles over all key
//    blocks and R = V - e^g Z, publishes R (barrier 2), forms v_new = A' R and the
//    gated v_new e^{g_last - g}, publishes them (barrier 3), and updates its state
//    rows with K^T v_gated, the decay e^{g_last} folded into the accumulator.
//  * output wave (w >= K/32) owns the same row tiles: after barrier 1 it forms
//    q h (the inter-chunk term); after barrier 3 it adds P v_new (the intra-chunk
//    term, P from the prep kernel) and stores its rows.
// One chain wave and one output wave share each SIMD. Each chunk's K is staged
// once in LDS (double buffered), prefetched one chunk ahead like every other
// operand; accumulations are split over independent accumulators.
// ---------------------------------------------------------------------------
template <int K, typename Tin>
struct ChainOps {
  using P = Prec<Tin>;
  static constexpr int NW = K / 32;
  static constexpr int RT = 4 / NW;
  typename P::Cmp a[RT][2];  // A' rows of my row tiles, per token block
  f32x4 v[RT];               // V at my rows, this slice's columns
  f32x4 eg[RT], egl[RT];     // e^g and e^{g_last - g} at my rows
  float dL;                  // e^{g_last}
};

template <int K, typename Tin>
struct OutOps {
  using P = Prec<Tin>;
  static constexpr int NW = K / 32;
  static constexpr int RT = 4 / NW;
  typename P::In q[RT][NW];   // q rows of my row tiles, per key block
  typename P::Cmp p[RT][2];   // P rows of my row tiles, per token block
  f32x4 eg[RT];               // e^g at my rows (D layout)
};

template <int K, int V, typename Tin, typename Tout>
__global__ __launch_bounds__(K / 32 * 128) void scan_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v, Tout* __restrict__ o, int H,
    float scale, int n_seqs, int T_eq, int ncs_eq, int total_tokens, int n_chunks, const int32_t* __restrict__ cu,
    const float* __restrict__ h0, float* __restrict__ ht, float* __restrict__ pool, int64_t pool_slots,
    const int32_t* __restrict__ slots, ChunkWs ws) {
  using P = Prec<Tin>;
  using Cmp = typename P::Cmp;
  using Stage = typename P::Stage;
  constexpr int NW = K / 32;
  constexpr int RT = 4 / NW;
  constexpr int NSL = V / 16;
  constexpr int NT = NW * 128;                              // threads
  constexpr int SK = K + (sizeof(Stage) == 2 ? 16 : 4);     // LDS row stride of the staged K
  constexpr int KSEG = 16 / sizeof(Stage);                  // elements per 16-byte segment
  constexpr int KLD = kChunk * K / KSEG / NT;               // 16-byte segments each thread stages
  __shared__ __attribute__((aligned(16))) Stage sK[2][kChunk][SK];
  __shared__ u32x4 sH[NW][2][64];        // state blocks (B operands, two planes)
  __shared__ u32x4 sR[2][2][64];         // R per token block (B operand)
  __shared__ u32x4 sV[2][2][2][64];      // [token block][v_new | gated v_new][plane][lane]

  // Workgroups of one (sequence, head) share an XCD (blockIdx % 8) and its L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, rest = bid >> 3;
  const int slice = rest % NSL;
  const int pair = (rest / NSL) * 8 + xcd;
  if (pair >= n_seqs * H) return;
  const int seq = pair / H, h = pair % H;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const bool chain = wv < NW;
  const int w = chain ? wv : wv - NW;
  const int lg = lane >> 4, lc = lane & 15;
  const int vcol = slice * 16 + lc;
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

  // K staging: every thread loads KLD 16-byte segments of the chunk's K rows
  // (rows past the end are zeroed) and writes them into sK[buffer].
  struct KStage {
    u32x4 seg[KLD];
  };
  auto load_k = [&](KStage& st, int c_req) {
    const int c = min(c_req, nc - 1);
    const int t0 = start + kChunk * c;
    const int n = min(kChunk, len - kChunk * c);
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int idx = tid + NT * i;
      const int row = idx / (K / KSEG), col = (idx % (K / KSEG)) * KSEG;
      const int rowc = min(row, n - 1);
      st.seg[i] = *reinterpret_cast<const u32x4*>(k + (static_cast<int64_t>(t0 + rowc) * H + h) * K + col);
      if (row >= n) st.seg[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_k = [&](const KStage& st, int buf) {
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int idx = tid + NT * i;
      const int row = idx / (K / KSEG), col = (idx % (K / KSEG)) * KSEG;
      *reinterpret_cast<u32x4*>(&sK[buf][row][col]) = st.seg[i];
    }
  };

  if (nc > 0) {
    KStage k0;
    load_k(k0, 0);
    store_k(k0, 0);
  }
  __syncthreads();

  if (chain) {
    using Ops = ChainOps<K, Tin>;
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
    // State slice h[key][value] = S[value][key]: two accumulator tiles.
    f32x4 hs[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int k0 = 32 * w + 16 * tt + 4 * lg;
      hs[tt] = s_in ? *reinterpret_cast<const f32x4*>(s_in + static_cast<int64_t>(vcol) * K + k0) : zero4();
    }

    // Loads are unconditional (a chunk index past the end is clamped to the last
    // chunk, rows past a chunk's end to its last row and zeroed after the load)
    // so the wait counters can keep the next chunk's loads in flight.
    auto load = [&](Ops& op, KStage& st, int c_req) {
      load_k(st, c_req + 1);
      const int c = min(c_req, nc - 1);
      const int64_t ch = static_cast<int64_t>(chunk0 + c) * H + h;
      const int t0 = start + kChunk * c;
      const int n = min(kChunk, len - kChunk * c);
#pragma unroll
      for (int rho = 0; rho < RT; ++rho) {
        const int rt = w * RT + rho;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          op.a[rho][ks] = P::ld_cmp(ws.af + ch * (8 * 2 * kPlane) + (rt * 2 + ks) * 2 * kPlane, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rt + 4 * lg + r;
          const float x = ld_in(v + (static_cast<int64_t>(t0 + min(row, n - 1)) * H + h) * V + vcol);
          op.v[rho][r] = row < n ? x : 0.f;
        }
        op.eg[rho] = *reinterpret_cast<const f32x4*>(ws.gx + ch * 192 + 64 + 16 * rt + 4 * lg);
        op.egl[rho] = *reinterpret_cast<const f32x4*>(ws.gx + ch * 192 + 128 + 16 * rt + 4 * lg);
      }
      op.dL = ws.gx[ch * 192 + 64 + 63];
    };

    auto step = [&](const Ops& cur, const KStage& nk, int c) {
      const int buf = c & 1;
      // (1) publish this wave's state block
      const Cmp hown = P::cmp_tiles(hs[0], hs[1]);
      P::st_cmp(&sH[w][0][0], lane, hown);
      __syncthreads();
      store_k(nk, buf ^ 1);  // next chunk's K: its buffer was last read before this barrier
      // (2) Z = K h for my row tiles; R = V - e^g Z
      Cmp hb[NW];
#pragma unroll
      for (int kb = 0; kb < NW; ++kb) hb[kb] = P::ld_cmp(&sH[kb][0][0], lane);
#pragma unroll
      for (int rho = 0; rho < RT; ++rho) {
        const int rt = w * RT + rho;
        f32x4 zp[NW];
#pragma unroll
        for (int kb = 0; kb < NW; ++kb) zp[kb] = mma(P::in_lds(&sK[buf][16 * rt + lc][32 * kb], lg), hb[kb], zero4());
        f32x4 z = zp[0];
#pragma unroll
        for (int kb = 1; kb < NW; ++kb) z += zp[kb];
        P::st_tile(&sR[rt >> 1][0][0], lane, rt & 1, cur.v[rho] - cur.eg[rho] * z);
      }
      __syncthreads();
      // (3) v_new = A' R (A' is lower triangular: token block 1 only for row tiles 2, 3)
      const Cmp r0 = P::ld_cmp(&sR[0][0][0], lane);
#pragma unroll
      for (int rho = 0; rho < RT; ++rho) {
        const int rt = w * RT + rho;
        f32x4 vn = mma(cur.a[rho][0], r0, zero4());
        if (rt >= 2) vn += mma(cur.a[rho][1], P::ld_cmp(&sR[1][0][0], lane), zero4());
        P::st_tile(&sV[rt >> 1][0][0][0], lane, rt & 1, vn);
        P::st_tile(&sV[rt >> 1][1][0][0], lane, rt & 1, vn * cur.egl[rho]);
      }
      __syncthreads();
      // (4) h <- e^{g_last} h + K^T v_gated
      const Cmp vg0 = P::ld_cmp(&sV[0][1][0][0], lane);
      const Cmp vg1 = P::ld_cmp(&sV[1][1][0][0], lane);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int kt = 2 * w + tt;
        const f32x4 a0 = mma(P::in_lds_tr(&sK[buf][0][0], SK, 0, 16 * kt, lane), vg0, hs[tt] * cur.dL);
        const f32x4 a1 = mma(P::in_lds_tr(&sK[buf][0][0], SK, 32, 16 * kt, lane), vg1, zero4());
        hs[tt] = a0 + a1;
      }
    };

    Ops bufA, bufB;
    KStage kA, kB;
    if (nc > 0) load(bufA, kA, 0);
    for (int c = 0; c < nc; c += 2) {
      load(bufB, kB, c + 1);
      step(bufA, kA, c);
      if (c + 1 >= nc) break;
      load(bufA, kA, c + 2);
      step(bufB, kB, c + 1);
    }
    if (s_out) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int k0 = 32 * w + 16 * tt + 4 * lg;
        *reinterpret_cast<f32x4*>(s_out + static_cast<int64_t>(vcol) * K + k0) = hs[tt];
      }
    }
  } else {
    using Ops = OutOps<K, Tin>;
    auto load = [&](Ops& op, KStage& st, int c_req) {
      load_k(st, c_req + 1);
      const int c = min(c_req, nc - 1);
      const int64_t ch = static_cast<int64_t>(chunk0 + c) * H + h;
      const int t0 = start + kChunk * c;
      const int n = min(kChunk, len - kChunk * c);
#pragma unroll
      for (int rho = 0; rho < RT; ++rho) {
        const int rt = w * RT + rho;
        const int row = 16 * rt + lc;
        const int rowc = min(row, n - 1);
#pragma unroll
        for (int kb = 0; kb < NW; ++kb) {
          op.q[rho][kb] = P::in_row(q + (static_cast<int64_t>(t0 + rowc) * H + h) * K + 32 * kb, lg);
          if (row >= n) op.q[rho][kb] = P::in_zero();
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          op.p[rho][ks] = P::ld_cmp(ws.pf + ch * (8 * 2 * kPlane) + (rt * 2 + ks) * 2 * kPlane, lane);
        op.eg[rho] = *reinterpret_cast<const f32x4*>(ws.gx + ch * 192 + 64 + 16 * rt + 4 * lg);
      }
    };

    auto step = [&](const Ops& cur, const KStage& nk, int c) {
      const int buf = c & 1;
      const int t0 = start + kChunk * c;
      const int n = min(kChunk, len - kChunk * c);
      __syncthreads();
      store_k(nk, buf ^ 1);
      // (1) inter-chunk term s e^g (q h)
      Cmp hb[NW];
#pragma unroll
      for (int kb = 0; kb < NW; ++kb) hb[kb] = P::ld_cmp(&sH[kb][0][0], lane);
      f32x4 acc[RT];
#pragma unroll
      for (int rho = 0; rho < RT; ++rho) {
        f32x4 yp[NW];
#pragma unroll
        for (int kb = 0; kb < NW; ++kb) yp[kb] = mma(cur.q[rho][kb], hb[kb], zero4());
        f32x4 y = yp[0];
#pragma unroll
        for (int kb = 1; kb < NW; ++kb) y += yp[kb];
        acc[rho] = (scale * cur.eg[rho]) * y;
      }
      __syncthreads();
      __syncthreads();
      // (2) intra-chunk term P v_new; store
      const Cmp vn0 = P::ld_cmp(&sV[0][0][0][0], lane);
#pragma unroll
      for (int rho = 0; rho < RT; ++rho) {
        const int rt = w * RT + rho;
        f32x4 o1 = zero4();
        if (rt >= 2) o1 = mma(cur.p[rho][1], P::ld_cmp(&sV[1][0][0][0], lane), o1);  // P is causal
        acc[rho] = mma(cur.p[rho][0], vn0, acc[rho]) + o1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rt + 4 * lg + r;
          if (row < n) store_out(o + (static_cast<int64_t>(t0 + row) * H + h) * V + vcol, acc[rho][r]);
        }
      }
    };

    Ops bufA, bufB;
    KStage kA, kB;
    if (nc > 0) load(bufA, kA, 0);
    for (int c = 0; c < nc; c += 2) {
      load(bufB, kB, c + 1);
      step(bufA, kA, c);
      if (c + 1 >= nc) break;
      load(bufA, kA, c + 2);
      step(bufB, kB, c + 1);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: workspace layout and launch sequence.
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

WsLayout workspace_layout(int64_t max_chunks, int n_seqs, int H, int K, int V, bool in_f32) {
  (void)K;
  (void)V;
  (void)in_f32;
  const size_t nch = static_cast<size_t>(max_chunks) * H;
  WsLayout l{};
  size_t off = 0;
  l.af = off;
  off = align256(off + nch * 8 * 2 * kPlane);
  l.pf = off;
  off = align256(off + nch * 8 * 2 * kPlane);
  l.gx = off;
  off = align256(off + nch * 3 * kChunk * 4);
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
  ws.af = reinterpret_cast<uint8_t*>(b + l.af);
  ws.pf = reinterpret_cast<uint8_t*>(b + l.pf);
  ws.gx = reinterpret_cast<float*>(b + l.gx);
  ws.info = reinterpret_cast<int4*>(b + l.info);
  ws.seq_chunk0 = reinterpret_cast<int*>(b + l.seq_chunk0);
  return ws;
}

template <int K, int V, typename Tin, typename Tout>
static hipError_t launch_chunk_t(const ChunkArgs& a) {
  constexpr int NSL = V / 16;
  const bool varlen = a.cu_seqlens != nullptr;
  const int ncs_eq = varlen ? 0 : (a.T_eq + kChunk - 1) / kChunk;
  if (a.events[0]) (void)hipEventRecord(a.events[0], a.stream);
  if (varlen) {
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(256), 0, a.stream, a.cu_seqlens, a.n_seqs,
                       static_cast<int>(a.total_tokens), static_cast<int>(a.n_chunks), a.ws.seq_chunk0,
                       a.ws.info);
  }
  if (a.n_chunks > 0) {
    hipLaunchKernelGGL((prep_kernel<K, Tin>), dim3(static_cast<unsigned>(a.n_chunks), a.H), dim3(256), 0,
                       a.stream, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), a.g, a.beta, a.H,
                       a.scale, a.T_eq, ncs_eq, static_cast<int>(a.total_tokens), varlen ? a.ws.info : nullptr,
                       a.ws);
  }
  if (a.events[1]) (void)hipEventRecord(a.events[1], a.stream);
  const int64_t pairs = static_cast<int64_t>(a.n_seqs) * a.H;
  const int64_t blocks = 8 * NSL * ((pairs + 7) / 8);
  hipLaunchKernelGGL((scan_kernel<K, V, Tin, Tout>), dim3(static_cast<unsigned>(blocks)), dim3(K / 32 * 128), 0,
                     a.stream, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                     static_cast<const Tin*>(a.v), static_cast<Tout*>(a.o), a.H, a.scale, a.n_seqs, a.T_eq, ncs_eq,
                     static_cast<int>(a.total_tokens), static_cast<int>(a.n_chunks), a.cu_seqlens, a.h0, a.ht, a.pool,
                     a.pool_slots, a.slots, a.ws);
  const hipError_t err = hipGetLastError();
  if (a.events[2]) (void)hipEventRecord(a.events[2], a.stream);
  return err;
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

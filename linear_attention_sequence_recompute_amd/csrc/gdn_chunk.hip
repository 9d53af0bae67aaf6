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
// recompute_w_u, plus the parts of chunk_fwd_o that do not depend on the state.
// One workgroup (4 waves) per (chunk, head).
// ---------------------------------------------------------------------------
template <int K, int V, typename Tin>
__global__ __launch_bounds__(256) void prep_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                                                   const Tin* __restrict__ v, const float* __restrict__ g,
                                                   const float* __restrict__ beta, int H, float scale,
                                                   int T_eq, int ncs_eq, int total_tokens,
                                                   const int4* __restrict__ info, ChunkWs ws) {
  using P = Prec<Tin>;
  using In = typename P::In;
  using Cmp = typename P::Cmp;
  using Stage = typename P::Stage;
  __shared__ __attribute__((aligned(16))) Stage sKt[K][kLdt];  // K^T: [key][token]
  __shared__ __attribute__((aligned(16))) Stage sVt[V][kLdt];  // V^T: [value][token]
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
    constexpr int PR = K / 8;
    for (int id = tid; id < kChunk * PR; id += 256) {
      const int t = id / PR, c8 = (id % PR) * 8;
      const Tin* p = k + (static_cast<int64_t>(t0 + t) * H + h) * K + c8;
#pragma unroll
      for (int e = 0; e < 8; ++e) sKt[c8 + e][t] = P::to_stage(t < n ? ld_in(p + e) : 0.f);
    }
  }
  {
    constexpr int PR = V / 8;
    for (int id = tid; id < kChunk * PR; id += 256) {
      const int t = id / PR, c8 = (id % PR) * 8;
      const Tin* p = v + (static_cast<int64_t>(t0 + t) * H + h) * V + c8;
#pragma unroll
      for (int e = 0; e < 8; ++e) sVt[c8 + e][t] = P::to_stage(t < n ? ld_in(p + e) : 0.f);
    }
  }
  for (int idx = tid; idx < 64 * 64; idx += 256) sA[idx >> 6][idx & 63] = (idx >> 6) == (idx & 63) ? 1.f : 0.f;
  __syncthreads();

  auto row_in = [&](const Tin* base, int row, int kb) -> In {
    return row < n ? P::in_row(base + (static_cast<int64_t>(t0 + row) * H + h) * K + 32 * kb, lg) : P::in_zero();
  };

  // (3) L = StrictLower(diag(beta) K K^T * E): the 10 lower 16x16 tiles.
  for (int tix = w; tix < 10; tix += 4) {
    const int bi = tix == 0 ? 0 : tix < 3 ? 1 : tix < 6 ? 2 : 3;
    const int bj = tix - (bi * (bi + 1)) / 2;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) acc = mma(row_in(k, 16 * bi + lc, kb), row_in(k, 16 * bj + lc, kb), acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * bi + 4 * lg + r, j = 16 * bj + lc;
      sL[i][j] = j < i ? sb[i] * acc[r] * __expf(sg[i] - sg[j]) : 0.f;
    }
  }

  // (4) P = s (Q K^T) * E * M, computed transposed so that pairs of accumulator
  // tiles are directly the A operands of P; wave w owns output row tile w.
  {
    const int bi = w;
    for (int ks = 0; ks < 2; ++ks) {
      f32x4 d[2] = {zero4(), zero4()};
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int bt = 2 * ks + half;
        if (bt > bi) continue;
#pragma unroll
        for (int kb = 0; kb < K / 32; ++kb)
          d[half] = mma(row_in(k, 16 * bt + lc, kb), row_in(q, 16 * bi + lc, kb), d[half]);
        const int i = 16 * bi + lc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tp = 16 * bt + 4 * lg + r;
          d[half][r] = tp <= i ? scale * d[half][r] * __expf(sg[i] - sg[tp]) : 0.f;
        }
      }
      P::st_cmp(ws.pf + ch * (8 * 2 * kPlane) + (bi * 2 + ks) * 2 * kPlane, lane, P::cmp_tiles(d[0], d[1]));
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

  // (6) u = A diag(beta) V; wave w owns output row tile w (all value tiles).
  {
    constexpr int NVT = V / 16;
    f32x4 acc[NVT];
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) acc[vt] = zero4();
    const int nks = w >= 2 ? 2 : 1;  // A is lower triangular
    for (int ks = 0; ks < nks; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = 32 * ks + kappa(lg, e);
        x[e] = sA[16 * w + lc][m] * sb[m];
      }
      const Cmp a = P::cmp8(x);
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) acc[vt] = mma(a, P::in_lds(&sVt[16 * vt + lc][32 * ks], lg), acc[vt]);
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
      const Cmp b = P::cmp8(x);
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) acc[kt] = mma(P::in_lds(&sKt[16 * kt + lc][32 * ks], lg), b, acc[kt]);
    }
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb)
      P::st_cmp(ws.wf + ch * (K * 256) + (kb * 4 + w) * 2 * kPlane, lane, P::cmp_tiles(acc[2 * kb], acc[2 * kb + 1]));
  }

  // (8) K^T as A operands for the state update of the scan kernel.
  for (int idx = w; idx < (K / 16) * 2; idx += 4) {
    const int kt = idx >> 1, ks = idx & 1;
    P::st_in(ws.ktf + ch * (K * 128 * P::kInPlanes) + (kt * 2 + ks) * P::kInPlanes * kPlane, lane,
             P::in_lds(&sKt[16 * kt + lc][32 * ks], lg));
  }
}

// ---------------------------------------------------------------------------
// chunk_fwd_h with chunk_fwd_o fused: sequential over the chunks of one
// sequence, for one head and one slice of 16 * NSUB value columns.
// ---------------------------------------------------------------------------
template <int K, int V, int NSUB, typename Tin, typename Tout>
__global__ __launch_bounds__(K / 32 * 64) void scan_kernel(
    const Tin* __restrict__ q, Tout* __restrict__ o, int H, float scale, int n_seqs, int T_eq,
    int ncs_eq, int total_tokens, int n_chunks, const int32_t* __restrict__ cu, const float* __restrict__ h0,
    float* __restrict__ ht, float* __restrict__ pool, int64_t pool_slots, const int32_t* __restrict__ slots,
    ChunkWs ws) {
  using P = Prec<Tin>;
  using In = typename P::In;
  using Cmp = typename P::Cmp;
  using Tile = typename P::Tile;
  constexpr int NW = K / 32;  // waves; wave w owns key rows [32w, 32w + 32)
  constexpr int RT = 4 / NW;  // output row tiles each wave finishes
  constexpr int NSL = V / (16 * NSUB);
  __shared__ f32x4 sX[NW][4][NSUB][64];   // partial w h over this wave's key rows
  __shared__ f32x4 sY[NW][4][NSUB][64];   // partial q h
  __shared__ Tile sVn[4][NSUB][2][64];    // v_new and gated v_new, B-operand ready

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

    // (1) the state as the B operand of this wave's 32-key block
    Cmp hb[NSUB];
#pragma unroll
    for (int ns = 0; ns < NSUB; ++ns) hb[ns] = P::cmp_tiles(hs[ns][0], hs[ns][1]);

    // (2) partial w h and q h over this wave's key rows, all 64 chunk rows
    const uint8_t* wf = ws.wf + ch * (K * 256) + (w * 4) * 2 * kPlane;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const Cmp wfr = P::ld_cmp(wf + rt * 2 * kPlane, lane);
      const int row = 16 * rt + lc;
      const In qf = row < n ? P::in_row(q + (static_cast<int64_t>(t0 + row) * H + h) * K + 32 * w, lg) : P::in_zero();
#pragma unroll
      for (int ns = 0; ns < NSUB; ++ns) {
        sX[w][rt][ns][lane] = mma(wfr, hb[ns], zero4());
        sY[w][rt][ns][lane] = mma(qf, hb[ns], zero4());
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
        f32x4 vn, vg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          vn[r] = u[r] - x[r];
          vg[r] = vn[r] * __expf(gL - gr[r]);
          acc_o[rho][ns][r] = scale * __expf(gr[r]) * y[r];
        }
        sVn[rt][ns][0][lane] = P::tile(vn);
        sVn[rt][ns][1][lane] = P::tile(vg);
      }
    }
    __syncthreads();

    // (4) state update: h <- e^{g_last} h + K^T v_gated, the decay folded into
    // the accumulator before the products are added.
    const float dL = __expf(gL);
    const uint8_t* ktf = ws.ktf + ch * (K * 128 * P::kInPlanes);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int kt = 2 * w + tt;
      In kf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) kf[ks] = P::ld_in_frag(ktf + (kt * 2 + ks) * P::kInPlanes * kPlane, lane);
#pragma unroll
      for (int ns = 0; ns < NSUB; ++ns) {
        f32x4 acc = hs[ns][tt] * dL;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          acc = mma(kf[ks], P::cmp_from(sVn[2 * ks][ns][1][lane], sVn[2 * ks + 1][ns][1][lane]), acc);
        hs[ns][tt] = acc;
      }
    }

    // (5) o = inter + P v_new for this wave's row tiles
#pragma unroll
    for (int rho = 0; rho < RT; ++rho) {
      const int rt = w * RT + rho;
      const uint8_t* pf = ws.pf + ch * (8 * 2 * kPlane) + rt * 2 * 2 * kPlane;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks == 1 && rt < 2) continue;  // P is causal: columns >= 32 vanish for rows < 32
        const Cmp pfr = P::ld_cmp(pf + ks * 2 * kPlane, lane);
#pragma unroll
        for (int ns = 0; ns < NSUB; ++ns)
          acc_o[rho][ns] = mma(pfr, P::cmp_from(sVn[2 * ks][ns][0][lane], sVn[2 * ks + 1][ns][0][lane]), acc_o[rho][ns]);
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
  ws.wf = reinterpret_cast<uint8_t*>(b + l.wf);
  ws.ktf = reinterpret_cast<uint8_t*>(b + l.ktf);
  ws.uf = reinterpret_cast<float*>(b + l.uf);
  ws.pf = reinterpret_cast<uint8_t*>(b + l.pf);
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
  if (a.events[0]) (void)hipEventRecord(a.events[0], a.stream);
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
  if (a.events[1]) (void)hipEventRecord(a.events[1], a.stream);
  const int64_t pairs = static_cast<int64_t>(a.n_seqs) * a.H;
  const int64_t blocks = 8 * NSL * ((pairs + 7) / 8);
  hipLaunchKernelGGL((scan_kernel<K, V, NSUB, Tin, Tout>), dim3(static_cast<unsigned>(blocks)), dim3(K / 32 * 64),
                     0, a.stream, static_cast<const Tin*>(a.q), static_cast<Tout*>(a.o), a.H, a.scale, a.n_seqs,
                     a.T_eq, ncs_eq, static_cast<int>(a.total_tokens), static_cast<int>(a.n_chunks),
                     a.cu_seqlens, a.h0, a.ht, a.pool, a.pool_slots, a.slots, a.ws);
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

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
//  * scan_kernel, one workgroup per (sequence, head, one or two 16-column slices
//    of V): the sequential chunk loop of chunk_fwd_h with chunk_fwd_o fused into
//    it. Each chunk's K is staged once in LDS and serves K h, K^T (read
//    transposed) and the score matrix P = s (Q K^T) * E * M; v_new =
//    A' (V - e^g (K h)); the state lives in MFMA accumulators, the decay
//    e^{g_last} folded into the accumulator before K^T v_gated is added.
//    Per-chunk states and v_new never leave the chip;
//  * with few (sequence, head) pairs, the chunk-parallel form: summary_kernel
//    forms the affine state map of each segment of chunks (h -> M h + c), and
//    scan_kernel then runs every segment at once, each chain first carrying the
//    initial state through the maps of the segments before its own.
//
// Precision: q, k, v are exact in bf16 and enter the MFMA as one operand; every
// computed operand (A', K h residuals, h, v_new, P) enters as a bf16 hi + lo pair
// with fp32 accumulation, which keeps about 16 significant bits. Float32 inputs
// run the same code on the fp32 MFMA.
#include <algorithm>
#include <type_traits>

#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kPlane = 1024;  // bytes of one fragment plane (64 lanes x 16 bytes)
constexpr int kMaxSegments = 8;  // segments per sequence in the chunk-parallel form

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

hipError_t launch_chunk_schedule(const int32_t* cu, int n_seqs, int total_tokens, int cap, int* seq_chunk0,
                                 int4* info, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(256), 0, stream, cu, n_seqs, total_tokens, cap, seq_chunk0, info);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// chunk_fwd_h with chunk_fwd_o fused: sequential over the chunks of one
// sequence, for one head and one slice of 16 value columns. Three waves:
//
//  * the chain wave (wave 0) holds the slice's whole [K x 16] state in MFMA
//    accumulators and runs the recurrence with no barrier inside a step and no
//    global memory access: per chunk it publishes the state (as the B operands
//    of K h), forms Z = K h, R = V - e^g Z, v_new = A' R (publishing v_new), and
//    h <- e^{g_last} h + K^T (v_new e^{g_last - g}), the decay folded into the
//    accumulator;
//  * two output waves (waves 1 and 2, row tiles {0, 1} and {2, 3}) run one
//    chunk behind: o = s e^g (q h) + P v_new from the published state and v_new,
//    with q, P and e^g loaded a chunk ahead into registers. They also stage the
//    chain's inputs for the chunk after the current one (K, A', the V slice and
//    the gate vectors) into LDS with direct global-to-LDS loads.
// All three meet at one barrier per chunk; every LDS buffer is double buffered.
//
// The state's key channels are held in a permuted order: within key block kb
// (32 keys), accumulator row 4 g + r of tile 2 kb + odd is key 32 kb + 8 g +
// 4 odd + r. Then the 8 contraction values a lane contributes to K h (and q h)
// are 8 consecutive keys, one 16-byte load, and a lane's two tiles of a block
// are 8 consecutive keys of the state in memory.
// ---------------------------------------------------------------------------
// Waits for this wave's outstanding vector-memory operations (including the
// direct-to-LDS copies) and nothing else: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// A chunk's K tile in LDS: 64 rows of K elements in 16-byte segments; segment
// s of row r is stored at position s ^ (r & kMask) of the row, so that 16
// consecutive rows read at one logical segment hit 16 different bank groups.
template <int K, typename T>
struct KTile {
  static constexpr int kRowBytes = K * static_cast<int>(sizeof(T));
  static constexpr int kSegs = kRowBytes / 16;
  static constexpr int kMask = (kSegs < 16 ? kSegs : 16) - 1;
  static constexpr int kBytes = kChunk * kRowBytes;
  static constexpr int kDmaOps = kBytes / 1024;
  static constexpr int kRowsPerOp = 1024 / kRowBytes;
  __device__ static __forceinline__ int at(int row, int seg) { return row * kRowBytes + ((seg ^ (row & kMask)) << 4); }
};

// A operand of K h (or q h) in the permuted key order: row `row`, key block kb;
// lane group g contributes keys [32 kb + 8 g, 32 kb + 8 g + 8).
template <int K, typename Tin>
struct KFrag;

template <int K>
struct KFrag<K, __bf16> {
  using T = KTile<K, __bf16>;
  __device__ static __forceinline__ FragB row(const char* tile, int row, int kb, int g) {
    return FragB{as_bf16x8(*reinterpret_cast<const u32x4*>(tile + T::at(row, 4 * kb + g)))};
  }
  __device__ static __forceinline__ FragB global_row(const __bf16* p, int kb, int g) {
    return FragB{as_bf16x8(*reinterpret_cast<const u32x4*>(p + 32 * kb + 8 * g))};
  }
  // A operand of K^T v: rows are the 16 keys of state tile 2 kb + odd, the
  // contraction runs over tokens [32 tb, 32 tb + 32). ds_read_b64_tr_b16 gives
  // output lane j of a 16-lane group element j & 3 of source lane 4 e + (j >> 2)
  // as its element e, so source lane l of group g reads the 4 keys
  // 32 kb + 8 (l & 3) + 4 odd .. + 3 of token 32 tb + 4 g + (l >> 2) (+ 16).
  __device__ static __forceinline__ FragB tr(const char* tile, int tb, int kb, int odd, int lane) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const int g = lane >> 4, l = lane & 15;
    const int r0 = 32 * tb + 4 * g + (l >> 2), seg = 4 * kb + (l & 3);
    const char* p0 = tile + T::at(r0, seg) + 8 * odd;
    const char* p1 = tile + T::at(r0 + 16, seg) + 8 * odd;
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
    const u32x2 au = __builtin_bit_cast(u32x2, a), bu = __builtin_bit_cast(u32x2, b);
    return FragB{as_bf16x8(u32x4{au[0], au[1], bu[0], bu[1]})};
  }
};

template <int K>
struct KFrag<K, float> {
  using T = KTile<K, float>;
  __device__ static __forceinline__ FragF row(const char* tile, int row, int kb, int g) {
    const int s = 8 * kb + 2 * g;
    return FragF{*reinterpret_cast<const f32x4*>(tile + T::at(row, s)),
                 *reinterpret_cast<const f32x4*>(tile + T::at(row, s + 1))};
  }
  __device__ static __forceinline__ FragF global_row(const float* p, int kb, int g) {
    return FragF{*reinterpret_cast<const f32x4*>(p + 32 * kb + 8 * g),
                 *reinterpret_cast<const f32x4*>(p + 32 * kb + 8 * g + 4)};
  }
  __device__ static __forceinline__ FragF tr(const char* tile, int tb, int kb, int odd, int lane) {
    const int g = lane >> 4, c = lane & 15;
    const int key = 32 * kb + 8 * (c >> 2) + 4 * odd + (c & 3);
    const int seg = key >> 2, off = 4 * (key & 3);
    FragF f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f.a[e] = *reinterpret_cast<const float*>(tile + T::at(32 * tb + 4 * g + e, seg) + off);
      f.b[e] = *reinterpret_cast<const float*>(tile + T::at(32 * tb + 16 + 4 * g + e, seg) + off);
    }
    return f;
  }
};

// Copies a chunk's K rows into a KTile in LDS. kd covers the chunk: row r at
// byte r * row_bytes, rows past the chunk's end outside the descriptor (read
// as zeros). Copy j, lane i fills position i % kSegs of tile row
// j * kRowsPerOp + i / kSegs with the segment the swizzle puts there.
// A wave may issue a share of the copies: j0, j0 + js, ... (js divides kDmaOps).
template <int K, typename Tin, int js = 1>
__device__ __forceinline__ void dma_k_tile(const Buf& kd, uint32_t row_bytes, char* tile, int j0 = 0) {
  using KT = KTile<K, Tin>;
  const int lane = threadIdx.x & 63;
  const uint32_t lane_row = static_cast<uint32_t>(lane / KT::kSegs) * row_bytes;
#pragma unroll
  for (int jj = 0; jj < KT::kDmaOps; jj += js) {
    const int j = jj + j0;
    const int row = j * KT::kRowsPerOp + lane / KT::kSegs;
    const uint32_t seg = static_cast<uint32_t>((lane % KT::kSegs) ^ (row & KT::kMask));
    kd.to_lds16(tile + 1024 * j, lane_row + 16 * seg, static_cast<uint32_t>(j * KT::kRowsPerOp) * row_bytes);
  }
}

// Copies a [64][16] slice (16 consecutive columns of each of a chunk's rows,
// row r at byte r * row_bytes of vd) into LDS in row-major order.
template <typename Tin>
__device__ __forceinline__ void dma_v_slice(const Buf& vd, uint32_t row_bytes, Tin* tile) {
  constexpr int kOps = kChunk * 16 * sizeof(Tin) / 1024;
  constexpr int kPerRow = 16 * sizeof(Tin) / 16;  // 16-byte pieces per row
  const int lane = threadIdx.x & 63;
  const uint32_t voff = static_cast<uint32_t>(lane / kPerRow) * row_bytes + 16 * (lane % kPerRow);
#pragma unroll
  for (int j = 0; j < kOps; ++j)
    vd.to_lds16(reinterpret_cast<char*>(tile) + 1024 * j, voff, static_cast<uint32_t>(j * (64 / kPerRow)) * row_bytes);
}

// A operand of q h / q k^T from global memory, permuted key order (keys
// [32 kb + 8 g, +8) for lane group g): voff addresses the lane's row and key
// group, soff the row tile and key block.
__device__ __forceinline__ FragB buf_frag(const Buf& b, uint32_t voff, uint32_t soff, const __bf16*) {
  return FragB{as_bf16x8(b.load16(voff, soff))};
}
__device__ __forceinline__ FragF buf_frag(const Buf& b, uint32_t voff, uint32_t soff, const float*) {
  return FragF{__builtin_bit_cast(f32x4, b.load16(voff, soff)), __builtin_bit_cast(f32x4, b.load16(voff + 16, soff))};
}

// A computed-operand fragment from its two 16-byte planes (hi, lo or a, b).
__device__ __forceinline__ FragS cmp_planes(const u32x4& x, const u32x4& y, FragS) {
  return FragS{as_bf16x8(x), as_bf16x8(y)};
}
__device__ __forceinline__ FragF cmp_planes(const u32x4& x, const u32x4& y, FragF) {
  return FragF{__builtin_bit_cast(f32x4, x), __builtin_bit_cast(f32x4, y)};
}

// Index of A' (or P) tile (row tile rt, token block ks) among the 6 nonzero
// ones: (0, 0) (1, 0) (2, 0) (2, 1) (3, 0) (3, 1). The workspace holds these 6
// per (chunk, head), each as hi and lo planes.
__host__ __device__ __forceinline__ constexpr int a_tile(int rt, int ks) { return rt < 2 ? rt : 2 + 2 * (rt - 2) + ks; }
constexpr int kTileSetBytes = 6 * 2 * kPlane;

// V at rows 16 rt + 4 g + i (i < 4), column c of a [64][16] LDS tile, for lane
// (g, c): the accumulator layout. Read (v_raw) and widened to fp32 (v_wide)
// separately, so that the read can be issued a phase ahead of its use. For bf16
// one transposed read serves the four rows: source lane l of group g reads
// columns 4 (l & 3) .. + 3 of row 16 rt + 4 g + (l >> 2), and output lane c
// receives element c & 3 of source lane 4 i + (c >> 2) as its element i.
__device__ __forceinline__ u32x2 v_raw(const __bf16* tile, int rt, int lane) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const int g = lane >> 4, l = lane & 15;
  const __bf16* p = tile + (16 * rt + 4 * g + (l >> 2)) * 16 + 4 * (l & 3);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p)));
}
__device__ __forceinline__ f32x4 v_wide(const u32x2& u) {
  return f32x4{__builtin_bit_cast(float, u[0] << 16), __builtin_bit_cast(float, u[0] & 0xffff0000u),
               __builtin_bit_cast(float, u[1] << 16), __builtin_bit_cast(float, u[1] & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 v_raw(const float* tile, int rt, int lane) {
  const int g = lane >> 4, c = lane & 15;
  const float* p = tile + (16 * rt + 4 * g) * 16 + c;
  return f32x4{p[0], p[16], p[32], p[48]};
}
__device__ __forceinline__ f32x4 v_wide(const f32x4& x) { return x; }

// ---------------------------------------------------------------------------
// recompute_w_u, reduced to what the fused scan needs: the chunk-local gate
// sums and A' = A diag(beta), A = (I + L)^-1 with L = StrictLower(diag(beta)
// K K^T * E), plus the state-independent score matrix P of chunk_fwd_o.
// One workgroup (4 waves) per (chunk, head).
//
// The inverse is formed by 16 x 16 blocks: each wave inverts one diagonal block
// D_i = (I + L_ii)^-1 by forward substitution, then the blocks below the
// diagonal follow by distance d = i - j from it,
//   A_ij = -D_i (sum_{j <= k < i} L_ik A_kj),   A_jj = D_j,
// as 16 x 16 x 16 products on the fp32 MFMA.
// ---------------------------------------------------------------------------
// 16-deep fp32 product on v_mfma_f32_16x16x4f32: lane (g, c) supplies a =
// X[c][4 g + e] and b = Y[4 g + e][c] to instruction e.
__device__ __forceinline__ f32x4 mma16_f32(const f32x4& a, const f32x4& b, f32x4 acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = mfma_f32(a[e], b[e], acc);
  return acc;
}

template <int K, typename Tin>
__global__ __launch_bounds__(256) void prep_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                                                   const float* __restrict__ g, const float* __restrict__ beta,
                                                   int H, float scale, int T_eq, int ncs_eq, int total_tokens,
                                                   int n_chunks, const int4* __restrict__ info, ChunkWs ws) {
  using P = Prec<Tin>;
  using In = typename P::In;
  using KF = KFrag<K, Tin>;
  using KT = KTile<K, Tin>;
  constexpr int NKB = K / 32;
  constexpr int LDA = 68;  // row stride (floats) of the L / A tile: 16-byte aligned rows
  __shared__ __attribute__((aligned(1024))) char sK[KT::kBytes];  // the chunk's K (swizzled)
  __shared__ __attribute__((aligned(16))) float sLA[64][LDA];     // L; diagonal blocks become D_i
  __shared__ float sOff[6][16][17];                                 // A_ij below the diagonal
  __shared__ float sg[64], sb[64];

  // Workgroup -> (chunk, head): the 8 XCDs take workgroups round-robin; XCD x
  // takes chunk x of every group of 8 chunks and runs its heads back to back, so
  // that the workgroups in flight together read whole token rows of q and k and
  // each chunk's rows are read through one L2 (prep 18.1 rather than 18.4 us at
  // B = 1 H = 16 T = 4096, 184 rather than 193 at B = 4 H = 32 T = 8192). The
  // grid is padded to whole groups; the padding exits at once.
  const int r8 = static_cast<int>(blockIdx.x >> 3);
  const int c = (r8 / H) * 8 + static_cast<int>(blockIdx.x & 7), h = r8 % H;
  if (c >= n_chunks) return;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  auto off_block = [](int i, int j) { return i * (i - 1) / 2 + j; };  // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)

  // (0) the chunk's K into LDS, a quarter of the copies per wave (rows past
  // the end read as zeros); this wave's 16 rows of Q
  constexpr uint32_t ES = sizeof(Tin);
  const uint32_t row_k = static_cast<uint32_t>(H) * K * ES;
  const int64_t base = static_cast<int64_t>(t0) * H + h;
  {
    const Buf kd(k + base * K, (n - 1) * row_k + K * ES);
    dma_k_tile<K, Tin, 4>(kd, row_k, sK, w);
  }
  // Fragments (row block rb, token block ks) of P, numbered 2 rb + ks, that
  // this wave computes in (2): three, three, two and two tiles per wave.
  constexpr int kGrp[4][2] = {{0, 6}, {2, 5}, {4, -1}, {7, -1}};
  In qg[2][NKB];
  {
    const Buf qd(q + base * K, (n - 1) * row_k + K * ES);
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int grp = kGrp[w][gi];
      if (grp < 0) continue;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        qg[gi][kb] = buf_frag(qd, lc * row_k + 8 * lg * ES, 16 * (grp >> 1) * row_k + 32 * kb * ES, q);
    }
  }

  // (1) chunk-local inclusive cumsum of the log-gate; beta; the gate vectors g,
  // e^g and e^{g_last - g} the scan kernel applies.
  if (w == 0) {
    const int64_t gi = static_cast<int64_t>(t0 + lane) * H + h;
    const float a = lane < n ? g[gi] : 0.f;
    const float gs = wave_inclusive_scan(a);
    // g_last is the sum at the chunk's last row, and rows past the end repeat it
    // exactly: the scan reaches lane 63 by another order of additions than lane
    // n - 1, and e^{g_last - g} of the last rows, which dominate the state when
    // the gates forget fast, must come out as 1 where it is 1.
    const float glast = __shfl(gs, n - 1, 64);
    const float gl = lane < n ? gs : glast;
    sg[lane] = gl;
    sb[lane] = lane < n ? beta[gi] : 0.f;
    ws.gx[ch * 192 + lane] = gl;
    ws.gx[ch * 192 + 64 + lane] = __expf(gl);
    ws.gx[ch * 192 + 128 + lane] = __expf(glast - gl);
  }
  wait_vmem();
  __syncthreads();

  // (2) L = StrictLower(diag(beta) K K^T * E) and the score matrix of
  // chunk_fwd_o, P = s (Q K^T) * E * M (E_ij = e^{g_i - g_j}, M the inclusive
  // causal mask), by fragment of P: the tiles (rb, bt <= rb), bt = 2 ks + half,
  // are computed transposed, K_bt K_rb^T and K_bt Q_rb^T, so that a pair of
  // accumulator tiles is directly the A operand of P and each element's E
  // serves both. Lane (g, c) then holds 4 consecutive columns j of row
  // i = 16 rb + c: L is written whole (zeros on and above the diagonal), one
  // 16-byte store per tile. Elements are computed and then selected (no branch).
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int grp = kGrp[w][gi];
    if (grp < 0) continue;
    const int rb = grp >> 1, ks = grp & 1;
    const int i = 16 * rb + lc;
    const float g_i = sg[i], b_i = sb[i];
    In kr[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) kr[kb] = KF::row(sK, i, kb, lg);
    f32x4 pt[2] = {zero4(), zero4()};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int bt = 2 * ks + half;
      if (bt > rb) continue;
      f32x4 lp[NKB], pp[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const In kt = KF::row(sK, 16 * bt + lc, kb, lg);
        lp[kb] = mma(kt, kr[kb], zero4());
        pp[kb] = mma(kt, qg[gi][kb], zero4());
      }
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb) {
        lp[0] += lp[kb];
        pp[0] += pp[kb];
      }
      const f32x4 g_j = *reinterpret_cast<const f32x4*>(&sg[16 * bt + 4 * lg]);
      f32x4 lv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * bt + 4 * lg + r;
        const float e = __expf(g_i - g_j[r]);
        const float xl = b_i * lp[0][r] * e, xp = scale * pp[0][r] * e;
        lv[r] = j < i ? xl : 0.f;
        pt[half][r] = j <= i ? xp : 0.f;
      }
      *reinterpret_cast<f32x4*>(&sLA[i][16 * bt + 4 * lg]) = lv;
    }
    P::st_cmp(ws.pf + ch * kTileSetBytes + a_tile(rb, ks) * 2 * kPlane, lane, P::cmp_tiles(pt[0], pt[1]));
  }
  __syncthreads();

  // (3) D_w = (I + L_ww)^-1 by forward substitution, rows of L_ww from
  // registers: the four lanes (j, part) of column j are adjacent; lane part
  // keeps rows [4 part, 4 part + 4) of column j. Row i of (I + L) D = I gives
  // D[i][j] = -sum_m L[i][m] D[m][j] (L[i][m] = 0 for m >= i, and D[m][j] not
  // yet known is 0); the four parts are added by quad permutations.
  {
    const int j = lane >> 2, part = lane & 3;
    f32x4 lrow[15];
#pragma unroll
    for (int i = 1; i < 16; ++i) lrow[i - 1] = *reinterpret_cast<const f32x4*>(&sLA[16 * w + i][16 * w + 4 * part]);
    f32x4 a;
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = (4 * part + r == j) ? 1.f : 0.f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      float s = (lrow[i - 1][0] * a[0] + lrow[i - 1][1] * a[1]) + (lrow[i - 1][2] * a[2] + lrow[i - 1][3] * a[3]);
      s += quad_xor1(s);
      s += quad_xor2(s);
      if (part == (i >> 2) && i > j) a[i & 3] = -s;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sLA[16 * w + 4 * part + r][16 * w + j] = a[r];
  }
  __syncthreads();

  // (4) the blocks below the diagonal, distance 1, 2, 3 (waves 0..3 - d)
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
        x = mma16_f32(lik, akj, x);
      }
      const f32x4 di = *reinterpret_cast<const f32x4*>(&sLA[16 * ib + lc][16 * ib + 4 * lg]);
      const f32x4 y = mma16_f32(di, x, zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) sOff[off_block(ib, jb)][4 * lg + r][lc] = -y[r];
    }
    __syncthreads();
  }

  // (5) A' = A diag(beta) as A operands: wave w stores row tile w, token blocks
  // 0 and, for row tiles 2 and 3, 1 (the other blocks are zero).
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (ks > 0 && w < 2) continue;  // zero, and never read
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int m = 32 * ks + kappa(lg, e);
      const int mb = m >> 4;
      const float av = mb == w ? sLA[16 * w + lc][m] : mb < w ? sOff[off_block(w, mb)][lc][m & 15] : 0.f;
      x[e] = av * sb[m];
    }
    P::st_cmp(ws.af + ch * kTileSetBytes + a_tile(w, ks) * 2 * kPlane, lane, P::cmp8(x));
  }
}

// LDS of one scan workgroup as one chain sees it, each buffer a separate
// __shared__ array so that the compiler can tell the direct-to-LDS copies from
// the exchange buffers (and does not make LDS reads wait for unrelated copies).
// K, A' and the gate vectors are shared by the NCH chains of a workgroup; the V
// slice, the published state and v_new are the chain's own.
template <int K, typename Tin, int NCH>
struct ScanSmem {
  static constexpr int NKB = K / 32;
  // The output waves' q tile with the gate vectors (kQLds) and P tiles
  // (kPLds) are staged in LDS by the producer where they fit: both for bf16
  // inputs and one chain per workgroup, q alone for two chains; otherwise the
  // output waves load them into registers a chunk ahead.
  static constexpr bool kQLds = sizeof(Tin) == 2;
  static constexpr bool kPLds = sizeof(Tin) == 2 && NCH == 1;
  static constexpr int kQBytes = kQLds ? KTile<K, Tin>::kBytes : 16;
  static constexpr int kQBufs = kQLds ? 2 : 1;
  static constexpr int kPTiles = kPLds ? 6 : 1;
  static constexpr int kPBufs = kPLds ? 2 : 1;
  char (*k)[KTile<K, Tin>::kBytes];  // [2] K tiles (swizzled), chain
  char (*a)[6][2 * kPlane];          // [2] A' tiles, two planes each, chain
  Tin (*v)[kChunk * 16];             // [2] V slice [token][16], chain
  float (*gx)[3 * kChunk];           // [2] g, e^g, e^{g_last - g}, chain
  char (*h)[NKB][2 * kPlane];        // [2] published state (B operands)
  f32x4 (*vn)[4][64];                // [2] published v_new tiles
  char (*qt)[kQBytes];               // [2] q tiles (swizzled like K), output waves
  char (*pt)[kPTiles][2 * kPlane];   // [2] P tiles, output waves
  float (*go)[3 * kChunk];           // [2] gate vectors, output waves
  char* fold[2];                     // map halves being folded (before the first chunk)
  char* sink;                        // 256 bytes nobody reads (L2 warming copies land there)
};

// A segment map M_j (K x K) as the A operands of the fold h <- M_j h + c_j:
// fragment (key block kb, state tile t) of two planes (hi, lo), lane (g, c)
// holding row krow(t, c) of M_j (the state tile's permuted key order) at
// columns 32 kb + 8 g .. + 7. Stored [kb][t][plane][64 lanes][16 bytes], so
// that the key blocks of one half of the contraction are contiguous (they are
// copied into LDS and folded half a map at a time).
template <int K>
struct MapFrag {
  static constexpr int NKB = K / 32;
  static constexpr int kBytes = NKB * 2 * NKB * 2 * kPlane;  // = K * K * 4
  static constexpr int kHalfBytes = kBytes / 2;
  __host__ __device__ static constexpr int at(int kb, int t) { return (kb * 2 * NKB + t) * 2 * kPlane; }
};

struct ScanSeq {
  int seq, h, slice, start, len, chunk0, nc;
};

// The chain wave. Its state slice starts from rows [lc][key] of s_in (zeros if
// null; if ident >= 0, the columns ident .. ident + 15 of the identity, which
// makes the final state those columns of the chunks' linear map), is then
// carried through n_fold segment maps (h <- M_j h + c_j: M_j from the LDS
// halves sm.fold the producer stages, this slice's c_j^T rows [lc][key] at
// fc + j fstride), and
// ends in s_out (if not null; rows [lc][key], or with out_t, for map columns,
// the split fragments of MapFrag at s_out). PUB: publish the state and v_new
// for output waves.
template <int K, int V, typename Tin, int NCH, bool PUB = true>
__device__ __forceinline__ void scan_chain(const ScanSmem<K, Tin, NCH>& sm, const ScanSeq& sq,
                                           const float* s_in, float* s_out, int ident,  // may alias
                                           bool out_t = false, const float* __restrict__ fc = nullptr,
                                           int n_fold = 0, int64_t fstride = 0) {
  using P = Prec<Tin>;
  using In = typename P::In;
  using Cmp = typename P::Cmp;
  using KF = KFrag<K, Tin>;
  constexpr int NKB = K / 32;
  const int lane = threadIdx.x & 63, lg = lane >> 4, lc = lane & 15;

  // State slice: tile 2 kb + odd, lane (g, c) holds keys 32 kb + 8 g + 4 odd + r
  // of value column c (S[c][key] in memory: 8 consecutive floats per block).
  f32x4 hs[2 * NKB];
#pragma unroll
  for (int t = 0; t < 2 * NKB; ++t) {
    const int key0 = 32 * (t >> 1) + 8 * lg + 4 * (t & 1);
    hs[t] = s_in ? *reinterpret_cast<const f32x4*>(s_in + lc * K + key0) : zero4();
    if (ident >= 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (key0 + r == ident + lc) hs[t][r] = 1.f;
    }
  }
  // The maps of the segments before this one, h <- M_j h + c_j, on the MFMA like
  // K h (A operand: map fragments, split hi + lo by the summary; B operand: the
  // state split), half a map (half the key blocks) at a time from the LDS
  // buffers the producer fills, one barrier per half. (The chunk-parallel form
  // runs for bf16 inputs only.)
  if (std::is_same<Tin, __bf16>::value && n_fold > 0) {
    using MF = MapFrag<K>;
    __syncthreads();  // the first half is staged
    for (int j = 0; j < n_fold; ++j) {
      const float* cj = fc + j * fstride;
      f32x4 cv[2 * NKB];
#pragma unroll
      for (int t = 0; t < 2 * NKB; ++t) {
        const int key0 = 32 * (t >> 1) + 8 * lg + 4 * (t & 1);
        cv[t] = *reinterpret_cast<const f32x4*>(cj + lc * K + key0);
      }
      Cmp hb[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) hb[kb] = P::cmp_tiles(hs[2 * kb], hs[2 * kb + 1]);
#pragma unroll
      for (int t = 0; t < 2 * NKB; ++t) hs[t] = zero4();
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const char* buf = sm.fold[hh];
#pragma unroll
        for (int kl = 0; kl < NKB / 2; ++kl) {
          const int kb = hh * (NKB / 2) + kl;
#pragma unroll
          for (int t = 0; t < 2 * NKB; ++t) {
            const Cmp am = P::ld_cmp(buf + MF::at(kl, t), lane);
#pragma unroll
            for (int u = 0; u < Terms<Cmp, Cmp>::n; ++u) hs[t] = term(am, hb[kb], hs[t], u);
          }
        }
        __syncthreads();  // this half is consumed; the next one is staged
      }
#pragma unroll
      for (int t = 0; t < 2 * NKB; ++t) hs[t] += cv[t];
    }
  }
  if (ident >= 0) {
    // a map column: the chunks' V enters as zeros (the producer leaves this
    // chain's V buffers alone)
#pragma unroll
    for (int b = 0; b < 2; ++b)
      for (int i = lane; i < kChunk * 16 * static_cast<int>(sizeof(Tin)) / 16; i += 64)
        reinterpret_cast<u32x4*>(sm.v[b])[i] = u32x4{0u, 0u, 0u, 0u};
  }
  constexpr int NZ = Terms<In, Cmp>::n;   // MFMA terms of K h and K^T v
  constexpr int NA = Terms<Cmp, Cmp>::n;  // MFMA terms of A' R
  using VRaw = decltype(v_raw(sm.v[0], 0, 0));
  __syncthreads();  // the first chunk's inputs are staged

  // One chunk step from state hs to hd; the LDS buffer index B is a
  // compile-time constant. hs is split into the B operands of K h in place,
  // after the decayed state e^{g_last} h (the update's accumulator) is formed.
  auto step = [&](auto B, f32x4 (&hs)[2 * NKB], f32x4 (&hd)[2 * NKB]) {
    constexpr int b = decltype(B)::value;
    const char* kt = sm.k[b];
    // LDS reads are issued one phase ahead of their use; scheduling barriers
    // keep each phase's reads, MFMAs and VALU work together.
    // (0) reads for (1): K rows of row tiles 0, 1, and e^{g_last}
    In kf[4][NKB];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) kf[rt][kb] = KF::row(kt, 16 * rt + lc, kb, lg);
    const float dL = sm.gx[b][64 + 63];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2 * NKB; ++t) hd[t] = hs[t] * dL;

    // (1) the state as the B operands of K h, one key block at a time; Z = K h
    // for row tiles 0, 1 (accumulators split by key-block parity for
    // independent chains); reads for (2): K rows of row tiles 2, 3, V, e^g
#pragma unroll
    for (int rt = 2; rt < 4; ++rt)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) kf[rt][kb] = KF::row(kt, 16 * rt + lc, kb, lg);
    Cmp hb[NKB];
    f32x4 z[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) z[rt][0] = z[rt][1] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      hb[kb] = P::cmp_tiles(hs[2 * kb], hs[2 * kb + 1]);
#pragma unroll
      for (int t = 0; t < NZ; ++t)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) z[rt][kb & 1] = term(kf[rt][kb], hb[kb], z[rt][kb & 1], t);
    }
    VRaw vr[4];
    f32x4 eg[4], egl[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      vr[rt] = v_raw(sm.v[b], rt, lane);
      eg[rt] = *reinterpret_cast<const f32x4*>(&sm.gx[b][64 + 16 * rt + 4 * lg]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // (2) Z for row tiles 2, 3, with R = V - e^g Z of row tiles 0, 1 under it;
    // reads for (3): A', e^{g_last - g}
    Cmp af[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) af[i] = P::ld_cmp(sm.a[b][i], lane);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) egl[rt] = *reinterpret_cast<const f32x4*>(&sm.gx[b][128 + 16 * rt + 4 * lg]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int t = 0; t < NZ; ++t)
#pragma unroll
        for (int rt = 2; rt < 4; ++rt) z[rt][kb & 1] = term(kf[rt][kb], hb[kb], z[rt][kb & 1], t);
    const Cmp rb0 = P::cmp_tiles(v_wide(vr[0]) - eg[0] * (z[0][0] + z[0][1]),
                                 v_wide(vr[1]) - eg[1] * (z[1][0] + z[1][1]));
    __builtin_amdgcn_sched_barrier(0);

    // (3) v_new = A' R, token block 0 of all row tiles, with R of row tiles 2, 3
    // split under it; reads for (5): K^T fragments of token block 0
    In ktf[2 * NKB][2];
#pragma unroll
    for (int t = 0; t < 2 * NKB; ++t) ktf[t][0] = KF::tr(kt, 0, t >> 1, t & 1, lane);
    f32x4 acc[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) acc[i] = zero4();
#pragma unroll
    for (int t = 0; t < NA; ++t)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = term(af[a_tile(rt, 0)], rb0, acc[rt], t);
    const Cmp rb1 = P::cmp_tiles(v_wide(vr[2]) - eg[2] * (z[2][0] + z[2][1]),
                                 v_wide(vr[3]) - eg[3] * (z[3][0] + z[3][1]));
    __builtin_amdgcn_sched_barrier(0);

    // (4) token block 1 of row tiles 2, 3 (A' is lower triangular), with the
    // gated v_new of row tiles 0, 1 under it; reads for (6): K^T of token block 1
#pragma unroll
    for (int t = 0; t < 2 * NKB; ++t) ktf[t][1] = KF::tr(kt, 1, t >> 1, t & 1, lane);
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      acc[4] = term(af[a_tile(2, 1)], rb1, acc[4], t);
      acc[5] = term(af[a_tile(3, 1)], rb1, acc[5], t);
    }
    if constexpr (PUB) {
      sm.vn[b][0][lane] = acc[0];
      sm.vn[b][1][lane] = acc[1];
    }
    const Cmp gb0 = P::cmp_tiles(acc[0] * egl[0], acc[1] * egl[1]);
    __builtin_amdgcn_sched_barrier(0);

    // (5) h <- e^{g_last} h + K^T (v_new e^{g_last - g}), token block 0, with
    // the rest of v_new under it
#pragma unroll
    for (int t = 0; t < NZ; ++t)
#pragma unroll
      for (int i = 0; i < 2 * NKB; ++i) hd[i] = term(ktf[i][0], gb0, hd[i], t);
    const f32x4 vn2 = acc[2] + acc[4], vn3 = acc[3] + acc[5];
    if constexpr (PUB) {
      sm.vn[b][2][lane] = vn2;
      sm.vn[b][3][lane] = vn3;
    }
    const Cmp gb1 = P::cmp_tiles(vn2 * egl[2], vn3 * egl[3]);
    __builtin_amdgcn_sched_barrier(0);

    // (6) token block 1
#pragma unroll
    for (int t = 0; t < NZ; ++t)
#pragma unroll
      for (int i = 0; i < 2 * NKB; ++i) hd[i] = term(ktf[i][1], gb1, hd[i], t);
    // the state this step started from, for the output waves (read after the barrier)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      if constexpr (PUB) P::st_cmp(sm.h[b][kb], lane, hb[kb]);
    __syncthreads();
  };
  // The state alternates between two register sets (hs in, hx out), so no
  // copy is made between steps.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  f32x4 hx[2 * NKB];
  int c = 0;
  for (; c + 1 < sq.nc; c += 2) {
    step(I0{}, hs, hx);
    step(I1{}, hx, hs);
  }
  if (c < sq.nc) {
    step(I0{}, hs, hx);
#pragma unroll
    for (int i = 0; i < 2 * NKB; ++i) hs[i] = hx[i];
  }
  if (s_out && out_t) {
    // columns ident + lc of M_j as split fragments (MapFrag): element (row, m)
    // with row = key(t, lg, r) sits in fragment (m >> 5, t), lane
    // (g' = (m >> 3) & 3, c' = 4 lg + r), element m & 7
    using MF = MapFrag<K>;
    const int m = ident + lc;
    char* base = reinterpret_cast<char*>(s_out);
    const int lane_off = (((m >> 3) & 3) * 16 + 4 * lg) * 16 + (m & 7) * 2;
#pragma unroll
    for (int t = 0; t < 2 * NKB; ++t) {
      uint32_t h01, l01, h23, l23;
      split2(hs[t][0], hs[t][1], h01, l01);
      split2(hs[t][2], hs[t][3], h23, l23);
      const uint32_t hv[4] = {h01 & 0xffffu, h01 >> 16, h23 & 0xffffu, h23 >> 16};
      const uint32_t lv[4] = {l01 & 0xffffu, l01 >> 16, l23 & 0xffffu, l23 >> 16};
      char* f = base + MF::at(m >> 5, t) + lane_off;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<uint16_t*>(f + r * 16) = static_cast<uint16_t>(hv[r]);
        *reinterpret_cast<uint16_t*>(f + kPlane + r * 16) = static_cast<uint16_t>(lv[r]);
      }
    }
  } else if (s_out) {
#pragma unroll
    for (int t = 0; t < 2 * NKB; ++t) {
      const int key0 = 32 * (t >> 1) + 8 * lg + 4 * (t & 1);
      *reinterpret_cast<f32x4*>(s_out + lc * K + key0) = hs[t];
    }
  }
}

// Every global access below goes through a buffer descriptor of one chunk:
// base at its first row for this head, size ending at its last row, so rows
// past the end read as zeros (loads, copies) or are dropped (stores).
// Per-lane offsets are the same for every chunk.
template <int K, int V, typename Tin>
struct ScanIo {
  static constexpr uint32_t ES = sizeof(Tin);
  const ScanSeq& sq;
  int H;
  uint32_t row_k, row_v;  // bytes between tokens of q / k and of v
  __device__ ScanIo(const ScanSeq& s, int h_count)
      : sq(s), H(h_count), row_k(static_cast<uint32_t>(h_count) * K * ES), row_v(static_cast<uint32_t>(h_count) * V * ES) {}
  __device__ int rows(int c) const { return min(kChunk, sq.len - kChunk * c); }
  __device__ int64_t token0(int c) const { return static_cast<int64_t>(sq.start + kChunk * c); }
  __device__ int64_t chunk_head(int c) const { return static_cast<int64_t>(sq.chunk0 + c) * H + sq.h; }
  __device__ Buf qk(const Tin* base, int c) const {  // q or k rows of chunk c, this head
    return Buf(base + (token0(c) * H + sq.h) * K, (rows(c) - 1) * row_k + K * ES);
  }
};

// The producer wave: every direct-to-LDS copy. In the interval that ends with
// chain step c it stages the chains' inputs of chunk c + 1 (K, A' and the gate
// vectors once, each chain's V slice) and, where they are staged in LDS, the
// output waves' inputs of chunk c (q, P, the gate vectors); all copies have
// landed before the barrier.
// SUM: for the segment summary kernel (no output waves; the V slices are
// staged only if has_v, the workgroup's chains being map columns otherwise).
// Before the first chunk it copies the halves of the n_fold segment maps the
// chains fold (fragments at maps + j * map_stride bytes) into sm.fold, one
// half per barrier, a half ahead of the chains.
template <int K, int V, typename Tin, int NCH, bool SUM = false>
__device__ __forceinline__ void scan_producer(const ScanSmem<K, Tin, NCH> (&sms)[NCH], const ScanSeq& sq,
                                              const Tin* __restrict__ q, const Tin* __restrict__ k,
                                              const Tin* __restrict__ v, int H, const ChunkWs& ws,
                                              bool has_v = true, const char* maps = nullptr, int n_fold = 0,
                                              int64_t map_stride = 0) {
  using S = ScanSmem<K, Tin, NCH>;
  const S& sm = sms[0];
  const int lane = threadIdx.x & 63;
  const ScanIo<K, V, Tin> io(sq, H);
  // Rows past the chunk's end are zeros: they meet zero columns of A' and
  // zero rows of v_new (and are never stored).
  auto stage_chain = [&](int c, int b) {
    dma_k_tile<K, Tin>(io.qk(k, c), io.row_k, sm.k[b]);
    const int64_t ch = io.chunk_head(c);
    const Buf ad(ws.af + ch * kTileSetBytes, kTileSetBytes);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks > 0 && rt < 2) continue;
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
          ad.to_lds16(sm.a[b][a_tile(rt, ks)] + pl * kPlane, 16 * lane, (a_tile(rt, ks) * 2 + pl) * kPlane);
      }
    if (!SUM || has_v) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const Buf vd(v + (io.token0(c) * H + sq.h) * V + (sq.slice + j) * 16,
                     (io.rows(c) - 1) * io.row_v + 16 * io.ES);
        dma_v_slice<Tin>(vd, io.row_v, sms[j].v[b]);
      }
    }
    const Buf gd(ws.gx + ch * 192, 192 * 4);
    if (lane < 3 * kChunk / 4) gd.to_lds16(sm.gx[b], 16 * lane, 0);
  };
  auto stage_out = [&](int c, int b) {
    const int64_t ch = io.chunk_head(c);
    if constexpr (S::kQLds) {
      dma_k_tile<K, Tin>(io.qk(q, c), io.row_k, sm.qt[b]);
      const Buf gd(ws.gx + ch * 192, 192 * 4);
      if (lane < 3 * kChunk / 4) gd.to_lds16(sm.go[b], 16 * lane, 0);
    }
    if constexpr (S::kPLds) {
      const Buf pd(ws.pf + ch * kTileSetBytes, kTileSetBytes);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          if (tb > 0 && rt < 2) continue;
#pragma unroll
          for (int pl = 0; pl < 2; ++pl)
            pd.to_lds16(sm.pt[b][a_tile(rt, tb)] + pl * kPlane, 16 * lane, (a_tile(rt, tb) * 2 + pl) * kPlane);
        }
    }
  };
  // L2 prefetch of chunk c: one 4-byte read per 128-byte line of its K and q
  // rows, A', P and this workgroup's V slices, into registers nobody uses (an
  // empty asm consumes them an interval later, when they have long landed, so
  // the compiler keeps the loads and waits for them only there). The NG
  // workgroups of a (sequence, head) share an XCD and its L2, so each takes
  // 1 / NG of the shared lines (rows or lines s, s + NG, ...); the V lines
  // are its own (its NCH slices are adjacent, 16 NCH elements of a row, within
  // one line). Five loads whatever c is (lanes with nothing to read are out of
  // range).
  constexpr int NG = SUM ? (V / 16 + K / 16) / NCH : V / 16 / NCH;
  constexpr int kLinesRow = KTile<K, Tin>::kRowBytes / 128;  // lines per K or q row (>= 1)
  constexpr int kRowsPer = kChunk / NG;
  static_assert(kRowsPer * kLinesRow <= 64 && kTileSetBytes / 128 / NG <= 64, "one load per region");
  static_assert(16 * NCH * sizeof(Tin) <= 128, "a workgroup's V slices share one line per row");
  const int grp = sq.slice / NCH;
  uint32_t sink[5] = {0u, 0u, 0u, 0u, 0u};
  auto prefetch = [&](int c) {
    const bool in = c < sq.nc;
    const int64_t ch = io.chunk_head(in ? c : 0);
    const uint32_t rows = in ? static_cast<uint32_t>(io.rows(c)) : 0u;
    const uint32_t kq_bytes = rows ? (rows - 1) * io.row_k + K * io.ES : 0u;
    const uint32_t kq_off = lane < kRowsPer * kLinesRow
                                ? static_cast<uint32_t>(grp * kRowsPer + lane / kLinesRow) * io.row_k +
                                      128u * (lane % kLinesRow)
                                : 0xFFFFFFF0u;
    const int64_t row0 = (io.token0(in ? c : 0) * H + sq.h) * K;
    sink[0] = Buf(k + row0, kq_bytes).load4(kq_off);
    if constexpr (!SUM) sink[1] = Buf(q + row0, kq_bytes).load4(kq_off);
    const uint32_t set_bytes = in ? static_cast<uint32_t>(kTileSetBytes) : 0u;
    const uint32_t set_off =
        lane < kTileSetBytes / 128 / NG ? 128u * static_cast<uint32_t>(grp + NG * lane) : 0xFFFFFFF0u;
    sink[2] = Buf(ws.af + ch * kTileSetBytes, set_bytes).load4(set_off);
    if constexpr (!SUM) sink[3] = Buf(ws.pf + ch * kTileSetBytes, set_bytes).load4(set_off);
    const Buf vd(v + (io.token0(in ? c : 0) * H + sq.h) * V + sq.slice * 16,
                 rows ? (rows - 1) * io.row_v + 16 * io.ES : 0u);
    sink[4] = vd.load4((!SUM || has_v) ? static_cast<uint32_t>(lane) * io.row_v : 0xFFFFFFF0u);
  };
  auto consume = [&] { asm volatile("" ::"v"(sink[0]), "v"(sink[1]), "v"(sink[2]), "v"(sink[3]), "v"(sink[4])); };
  constexpr int kPrefetchOps = SUM ? 3 : 5;
  const int nc = sq.nc;
  if (nc > 0) stage_chain(0, 0);
  if (n_fold > 0) {
    using MF = MapFrag<K>;
    auto stage_half = [&](int hf) {  // half hf & 1 of map hf >> 1
      const Buf md(maps + (hf >> 1) * map_stride + (hf & 1) * MF::kHalfBytes, MF::kHalfBytes);
      char* dst = (hf & 1) ? sm.fold[1] : sm.fold[0];  // a select: an indexed member array would live in scratch
#pragma unroll
      for (int j = 0; j < MF::kHalfBytes / 1024; ++j) md.to_lds16(dst + 1024 * j, 16 * lane, 1024 * j);
    };
    // (the maps' lines are brought into L2 by output wave 1 meanwhile, so that
    // this wave's first wait covers the first chunk and the first half only)
    stage_half(0);
    wait_vmem();
    __syncthreads();
    for (int hf = 0; hf < 2 * n_fold; ++hf) {
      if (hf + 1 < 2 * n_fold) stage_half(hf + 1);
      wait_vmem();
      __syncthreads();
    }
  }
  wait_vmem();
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    if (c + 1 < nc) stage_chain(c + 1, (c + 1) & 1);
    if constexpr (!SUM && (S::kQLds || S::kPLds)) stage_out(c, c & 1);
    consume();  // the previous interval's prefetches (older than these copies)
    prefetch(c + 2);
    // the copies have landed; the prefetches, issued last, may still be in
    // flight (the count drains in issue order)
    __builtin_amdgcn_s_waitcnt(0x0F70 | kPrefetchOps);
    __syncthreads();
  }
  consume();
}

// Output wave OW (row tiles 2 OW and 2 OW + 1): in the interval that ends with
// chain step c it emits the rows of chunk c - 1, o = s e^g (q h) + P v_new,
// from the published state and v_new, for each of the workgroup's NCH slices
// (the q, P and e^g operands serve all of them).
template <int OW, int K, int V, typename Tin, typename Tout, int NCH>
__device__ __forceinline__ void scan_output(const ScanSmem<K, Tin, NCH> (&sms)[NCH], const ScanSeq& sq,
                                            const Tin* __restrict__ q, Tout* __restrict__ o, int H, float scale,
                                            const ChunkWs& ws, int n_fold = 0, const char* maps = nullptr,
                                            int64_t map_stride = 0) {
  using S = ScanSmem<K, Tin, NCH>;
  const S& sm0 = sms[0];
  using P = Prec<Tin>;
  using In = typename P::In;
  using Cmp = typename P::Cmp;
  using KF = KFrag<K, Tin>;
  constexpr int NKB = K / 32;
  constexpr int NTB = OW + 1;  // token blocks of P v_new for these row tiles
  const int lane = threadIdx.x & 63, lg = lane >> 4, lc = lane & 15;
  const ScanIo<K, V, Tin> io(sq, H);
  const uint32_t row_o = static_cast<uint32_t>(H) * V * sizeof(Tout);

  constexpr bool kQ = S::kQLds, kP = S::kPLds;
  // operands not staged in LDS, loaded into registers one chunk ahead (the
  // arrays of staged operands have one unused element)
  struct Regs {
    In q[kQ ? 1 : 2][kQ ? 1 : NKB];
    f32x4 eg[kQ ? 1 : 2];
    Cmp p[kP ? 1 : 2][kP ? 1 : NTB];
  };
  const uint32_t q_voff = static_cast<uint32_t>(lc) * io.row_k + 8 * lg * io.ES;
  auto load = [&](Regs& rg, int c) {
    const int64_t ch = io.chunk_head(c);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rt = 2 * OW + i;
      if constexpr (!kQ) {
        const Buf qd = io.qk(q, c);
        const Buf gd(ws.gx + ch * 192, 192 * 4);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) rg.q[i][kb] = buf_frag(qd, q_voff, 16 * rt * io.row_k + 32 * kb * io.ES, q);
        rg.eg[i] = __builtin_bit_cast(f32x4, gd.load16(4 * (64 + 16 * rt + 4 * lg), 0));
      }
      if constexpr (!kP) {
        const Buf pd(ws.pf + ch * kTileSetBytes, kTileSetBytes);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          const uint32_t so = a_tile(rt, tb) * 2 * kPlane;
          rg.p[i][tb] = cmp_planes(pd.load16(16 * lane, so), pd.load16(16 * lane, so + kPlane), Cmp{});
        }
      }
    }
  };

  // o rows of chunk c, for each slice, from the q fragments, P fragments and
  // e^g (from LDS buffer c & 1 or from rg) and the published state and v_new
  auto emit = [&](int c, const Regs& rg) {
    const int b = c & 1;
    In qf[2][NKB];
    Cmp pf[2][NTB];
    f32x4 eg[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rt = 2 * OW + i;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if constexpr (kQ)
          qf[i][kb] = KF::row(sm0.qt[b], 16 * rt + lc, kb, lg);
        else
          qf[i][kb] = rg.q[i][kb];
      }
      if constexpr (kQ)
        eg[i] = *reinterpret_cast<const f32x4*>(&sm0.go[b][64 + 16 * rt + 4 * lg]);
      else
        eg[i] = rg.eg[i];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        if constexpr (kP)
          pf[i][tb] = P::ld_cmp(sm0.pt[b][a_tile(rt, tb)], lane);
        else
          pf[i][tb] = rg.p[i][tb];
      }
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const S& sm = sms[j];
      const Buf od(o + (io.token0(c) * H + sq.h) * V + (sq.slice + j) * 16,
                   (io.rows(c) - 1) * row_o + 16 * sizeof(Tout));
      Cmp hb[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) hb[kb] = P::ld_cmp(sm.h[b][kb], lane);
      Cmp vb[NTB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) vb[tb] = P::cmp_tiles(sm.vn[b][2 * tb][lane], sm.vn[b][2 * tb + 1][lane]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rt = 2 * OW + i;
        f32x4 y = mma(qf[i][0], hb[0], zero4());
#pragma unroll
        for (int kb = 1; kb < NKB; ++kb) y = mma(qf[i][kb], hb[kb], y);
        f32x4 acc = (scale * eg[i]) * y;
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) acc = mma(pf[i][tb], vb[tb], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          od.store(static_cast<Tout>(acc[r]), (4 * lg + r) * row_o + lc * sizeof(Tout), 16 * rt * row_o);
      }
    }
  };

  // every line of the maps the chains fold into L2 (a 4-byte direct-to-LDS
  // read per 128-byte line, into a block nobody reads: no registers held), so
  // that the producer's half copies, a half ahead of the chains, hit L2; then
  // the barriers of the folds (two halves per map, one more before)
  if (OW == 1 && n_fold > 0) {
    using MF = MapFrag<K>;
    for (int j = 0; j < n_fold; ++j) {
      const Buf md(maps + j * map_stride, MF::kBytes);
#pragma unroll
      for (int i = 0; i < MF::kBytes / 128 / 64; ++i) md.to_lds4(sm0.sink, 128u * (64 * i + lane), 0);
    }
  }
  for (int hf = 0; n_fold > 0 && hf <= 2 * n_fold; ++hf) __syncthreads();
  const int nc = sq.nc;
  __syncthreads();
  if constexpr (kQ && kP) {
    const Regs none{};
    for (int c = 0; c < nc; ++c) {
      if (c > 0) emit(c - 1, none);
      __syncthreads();
    }
    if (nc > 0) emit(nc - 1, none);
  } else if (nc > 0) {
    // ping-pong register sets; the loads of chunk c go out at the start of
    // the interval that emits chunk c - 1
    Regs ra, rb;
    load(ra, 0);
    wait_vmem();
    __syncthreads();
    int c = 1;
    for (; c + 1 < nc; c += 2) {  // c odd
      load(rb, c);
      __builtin_amdgcn_sched_barrier(0);  // loads go out before the output work
      emit(c - 1, ra);
      wait_vmem();
      __syncthreads();
      load(ra, c + 1);
      __builtin_amdgcn_sched_barrier(0);
      emit(c, rb);
      wait_vmem();
      __syncthreads();
    }
    if (c < nc) {  // c == nc - 1: intervals nc - 1 and nc remain
      load(rb, c);
      __builtin_amdgcn_sched_barrier(0);
      emit(c - 1, ra);
      wait_vmem();
      __syncthreads();
      emit(c, rb);
    } else {  // c == nc: the last interval remains
      emit(c - 1, ra);
    }
  }
  wait_vmem();
}

// Threads of a scan workgroup: one chain wave per slice, two output waves and
// the producer wave.
template <int NCH>
constexpr int scan_threads() {
  return 64 * (NCH + 3);
}

// The chunks of (sequence, head) pair `pair`: first token, length, global
// index of its first chunk. A packed call whose offsets do not fit [0,
// total_tokens] or the chunk count gets an empty sequence (no access can leave
// the inputs or the workspace).
__device__ __forceinline__ ScanSeq seq_of(int pair, int H, int T_eq, int ncs_eq, int total_tokens, int n_chunks,
                                          const int32_t* __restrict__ cu, const ChunkWs& ws) {
  ScanSeq sq;
  sq.slice = 0;
  sq.seq = pair / H;
  sq.h = pair % H;
  if (cu) {
    sq.start = cu[sq.seq];
    sq.len = cu[sq.seq + 1] - sq.start;
    sq.chunk0 = ws.seq_chunk0[sq.seq];
    const int nc_want = (sq.len + kChunk - 1) / kChunk;
    if (sq.start < 0 || sq.len < 0 || sq.start > total_tokens - sq.len || sq.chunk0 < 0 ||
        sq.chunk0 > n_chunks - nc_want)
      sq.len = 0;
  } else {
    sq.start = sq.seq * T_eq;
    sq.len = T_eq;
    sq.chunk0 = sq.seq * ncs_eq;
  }
  sq.nc = (sq.len + kChunk - 1) / kChunk;
  return sq;
}

// Segments of the chunk-parallel form: segment 0 holds the first L0 chunks of a
// sequence, each later one L1 chunks, the last one whatever remains. A
// sequence of nc chunks has max(1, 1 + ceil((nc - L0) / L1)) segments, never
// more than n_seg (the grid's and the workspace's count, whatever the device
// copy of the offsets says); segment 0 exists even for an empty sequence, so
// that its initial state passes to its final state. The host picks L0 and L1
// (segment_lengths).
struct SegGeom {
  int n_seg, L0, L1;
  __device__ int count(int nc) const { return nc <= L0 ? 1 : min(n_seg, 1 + (nc - L0 + L1 - 1) / L1); }
  // restricts sq to segment `seg` (< count(sq.nc))
  __device__ void restrict(ScanSeq& sq, int seg) const {
    const int ns = count(sq.nc);
    const int c0 = seg == 0 ? 0 : L0 + (seg - 1) * L1;
    const int c1 = seg == ns - 1 ? sq.nc : min(sq.nc, seg == 0 ? L0 : L0 + seg * L1);
    sq.start += kChunk * c0;
    sq.chunk0 += c0;
    sq.len = max(0, min(sq.len - kChunk * c0, kChunk * (c1 - c0)));
    sq.nc = (sq.len + kChunk - 1) / kChunk;
  }
};

// Arguments every scan-side kernel takes.
template <typename Tin, typename Tout>
struct ScanArgs {
  const Tin* q;
  const Tin* k;
  const Tin* v;
  Tout* o;
  int H;
  float scale;
  int n_seqs, T_eq, ncs_eq, total_tokens, n_chunks;
  const int32_t* cu;
  const float* h0;  // h0 and ht may alias (in-place update)
  float* ht;
  float* pool;
  int64_t pool_slots;
  const int32_t* slots;
  SegGeom geo;
  ChunkWs ws;
};

// The sequence's initial (st_in) and final (st_out) state pages of head sq.h:
// a pool slot, or h0 / ht (null: zero start / not stored).
template <int K, int V, typename Tin, typename Tout>
__device__ __forceinline__ void state_pages(const ScanArgs<Tin, Tout>& a, const ScanSeq& sq, const float*& st_in,
                                            float*& st_out) {
  const int64_t page = static_cast<int64_t>(V) * K;
  st_in = nullptr;
  st_out = nullptr;
  if (a.pool) {
    const int s = a.slots[sq.seq];
    if (s > 0 && s < a.pool_slots) {
      st_in = a.pool + (static_cast<int64_t>(s) * a.H + sq.h) * page;
      st_out = a.pool + (static_cast<int64_t>(s) * a.H + sq.h) * page;
    }
  } else {
    if (a.h0) st_in = a.h0 + (static_cast<int64_t>(sq.seq) * a.H + sq.h) * page;
    if (a.ht) st_out = a.ht + (static_cast<int64_t>(sq.seq) * a.H + sq.h) * page;
  }
}

// One scan workgroup (pair, slices grp * NCH .., segment seg) over LDS sm:
// waves 0 .. NCH - 1 run the chains, the producer and two output waves the rest.
// NCH = 1: waves 0 chain, 1 producer, 2 and 3 output. NCH = 2: waves 0 and 1
// chains, 2 and 3 output, 4 producer. The waves of a workgroup are spread over
// the four SIMDs of its CU (waves 0..3 on four different ones, wave 4 beside
// wave 0), so each chain, which is bound by its own instruction issue, has a
// SIMD to itself or shares it with the producer, the lightest role.
//
// Chunk-parallel form (geo.n_seg > 1): segment 0 runs from the sequence's
// initial state and, when later segments exist, leaves its final state in
// ws.seg_state (their common starting point); segment j >= 1 starts from that
// state carried through the maps of segments 1 .. j - 1 (summary part of the
// first launch); only the sequence's last segment stores its final state.
template <int K, int V, typename Tin, typename Tout, int NCH>
__device__ __forceinline__ void scan_wg(const ScanSmem<K, Tin, NCH> (&sms)[NCH], const ScanArgs<Tin, Tout>& a,
                                        int pair, int grp, int seg) {
  ScanSeq sq = seq_of(pair, a.H, a.T_eq, a.ncs_eq, a.total_tokens, a.n_chunks, a.cu, a.ws);
  sq.slice = grp * NCH;  // the workgroup's first slice
  const float* st_in;
  float* st_out;
  state_pages<K, V>(a, sq, st_in, st_out);
  const int64_t page = static_cast<int64_t>(V) * K;
  const float* fold = nullptr;
  int n_fold = 0;
  if (a.geo.n_seg > 1) {
    const int ns = a.geo.count(sq.nc);
    if (seg >= ns) return;
    a.geo.restrict(sq, seg);
    float* mid = a.ws.seg_state + static_cast<int64_t>(pair) * page;
    if (seg > 0) {
      st_in = mid;
      fold = a.ws.seg_sum + static_cast<int64_t>(pair) * (a.geo.n_seg - 2) * (V + K) * K;
      n_fold = seg - 1;
    }
    if (seg != ns - 1) st_out = seg == 0 ? mid : nullptr;
  }

  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int kProducer = NCH == 1 ? 1 : 4;
  if (wv < NCH) {
    ScanSeq cs = sq;
    cs.slice = sq.slice + wv;
    const int64_t rows = static_cast<int64_t>(cs.slice) * 16 * K;
    const float* s_in = st_in ? st_in + rows : nullptr;
    float* s_out = st_out ? st_out + rows : nullptr;
    const float* fc = fold ? fold + rows : nullptr;
    const int64_t fstride = static_cast<int64_t>(V + K) * K;
    if (wv == 0)
      scan_chain<K, V, Tin, NCH>(sms[0], cs, s_in, s_out, -1, false, fc, n_fold, fstride);
    else
      scan_chain<K, V, Tin, NCH>(sms[NCH - 1], cs, s_in, s_out, -1, false, fc, n_fold, fstride);
  } else if (wv == kProducer) {
    const char* maps = fold ? reinterpret_cast<const char*>(fold + static_cast<int64_t>(V) * K) : nullptr;
    scan_producer<K, V, Tin, NCH>(sms, sq, a.q, a.k, a.v, a.H, a.ws, true, maps, n_fold,
                                  static_cast<int64_t>(V + K) * K * 4);
  } else {
    const char* maps = fold ? reinterpret_cast<const char*>(fold + static_cast<int64_t>(V) * K) : nullptr;
    if (wv == 2)
      scan_output<0, K, V, Tin, Tout, NCH>(sms, sq, a.q, a.o, a.H, a.scale, a.ws, n_fold);
    else
      scan_output<1, K, V, Tin, Tout, NCH>(sms, sq, a.q, a.o, a.H, a.scale, a.ws, n_fold, maps,
                                           static_cast<int64_t>(V + K) * K * 4);
  }
}

// A segment's affine state map, h_out = M_j h_in + c_j (the chunk step is
// linear in h): workgroup (pair, segment j >= 1, 4 slices) runs the segment's
// chain with four chain waves (one per SIMD) and the producer: slices of c_j
// start from zero with the chunks' V, slices of M_j start from identity
// columns with V = 0. Page (pair, j - 1) of the workspace holds c_j^T as rows
// [v][key] (float32), then M_j as split A-operand fragments (MapFrag). Only
// maps that a later segment of the sequence folds are formed (not the last
// segment's).
template <int K, int V, typename Tout>
__device__ __forceinline__ void summary_wg(const ScanSmem<K, __bf16, 4> (&sms)[4],
                                           const ScanArgs<__bf16, Tout>& a, int pair, int grp, int seg) {
  constexpr int NCH = 4;
  constexpr int NSL = V / 16;
  ScanSeq sq = seq_of(pair, a.H, a.T_eq, a.ncs_eq, a.total_tokens, a.n_chunks, a.cu, a.ws);
  if (seg >= a.geo.count(sq.nc) - 1) return;  // no later segment folds this map
  a.geo.restrict(sq, seg);
  sq.slice = grp * NCH;
  const bool is_c = sq.slice < NSL;
  float* page = a.ws.seg_sum + (static_cast<int64_t>(pair) * (a.geo.n_seg - 2) + seg - 1) * (V + K) * K;

  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wv < NCH) {
    ScanSeq cs = sq;
    cs.slice = sq.slice + wv;
    // c rows [v][key]; columns m0 .. m0 + 15 of M_j into its split fragments
    const int ident = is_c ? -1 : (cs.slice - NSL) * 16;
    float* s_out = is_c ? page + static_cast<int64_t>(cs.slice) * 16 * K : page + static_cast<int64_t>(V) * K;
    if (wv == 0)
      scan_chain<K, V, __bf16, NCH, false>(sms[0], cs, nullptr, s_out, ident, !is_c);
    else if (wv == 1)
      scan_chain<K, V, __bf16, NCH, false>(sms[1], cs, nullptr, s_out, ident, !is_c);
    else if (wv == 2)
      scan_chain<K, V, __bf16, NCH, false>(sms[2], cs, nullptr, s_out, ident, !is_c);
    else
      scan_chain<K, V, __bf16, NCH, false>(sms[3], cs, nullptr, s_out, ident, !is_c);
  } else {
    scan_producer<K, V, __bf16, NCH, true>(sms, sq, nullptr, a.k, a.v, a.H, a.ws, is_c);
  }
}

// The LDS of a scan workgroup, as separate __shared__ arrays (so that the
// compiler can tell the direct-to-LDS copies from the exchange buffers and does
// not make LDS reads wait for unrelated copies), and its view per chain.
#define GDN_SCAN_LDS(K, Tin, NCH)                                                         \
  using S = ScanSmem<K, Tin, NCH>;                                                        \
  constexpr int NKB = K / 32;                                                             \
  __shared__ __attribute__((aligned(1024))) char lds_k[2][KTile<K, Tin>::kBytes];         \
  __shared__ __attribute__((aligned(1024))) char lds_a[2][6][2 * kPlane];                 \
  __shared__ __attribute__((aligned(1024))) Tin lds_v[NCH][2][kChunk * 16];               \
  __shared__ __attribute__((aligned(16))) float lds_gx[2][3 * kChunk];                    \
  __shared__ __attribute__((aligned(16))) char lds_h[NCH][2][NKB][2 * kPlane];            \
  __shared__ __attribute__((aligned(16))) f32x4 lds_vn[NCH][2][4][64];                    \
  __shared__ __attribute__((aligned(1024))) char lds_qt[S::kQBufs][S::kQBytes];           \
  __shared__ __attribute__((aligned(1024))) char lds_pt[S::kPBufs][S::kPTiles][2 * kPlane]; \
  __shared__ __attribute__((aligned(16))) float lds_go[S::kQBufs][3 * kChunk];            \
  S sms[NCH];                                                                             \
  _Pragma("unroll") for (int j = 0; j < NCH; ++j) sms[j] =                                \
      S{lds_k, lds_a, lds_v[j], lds_gx, lds_h[j], lds_vn[j], lds_qt, lds_pt, lds_go,      \
        {&lds_qt[0][0], &lds_h[0][0][0][0]}, &lds_pt[S::kPBufs - 1][S::kPTiles - 1][0]};    \
  static_assert(NCH == 1 || (sizeof(lds_qt) >= MapFrag<K>::kHalfBytes &&                  \
                             sizeof(lds_h) >= MapFrag<K>::kHalfBytes),                    \
                "a map half fits each fold buffer");

// The single-pass scan (geo.n_seg == 1) or, in the chunk-parallel form, the
// segments j >= 1 of every sequence at once (second launch).
// Workgroups of one (sequence, head) share an XCD (blockIdx % 8) and its L2.
template <int K, int V, typename Tin, typename Tout, int NCH>
__global__ __launch_bounds__(scan_threads<NCH>()) __attribute__((amdgpu_waves_per_eu(NCH, NCH))) void scan_kernel(
    ScanArgs<Tin, Tout> a) {
  static_assert(NCH == 1 || NCH == 2, "one or two chains per workgroup");
  GDN_SCAN_LDS(K, Tin, NCH)
  constexpr int NG = V / 16 / NCH;  // workgroups per (sequence, head, segment)
  const int bid = blockIdx.x;
  const int xcd = bid & 7, rest = bid >> 3;
  const int grp = rest % NG, r2 = rest / NG;
  const int nl = a.geo.n_seg > 1 ? a.geo.n_seg - 1 : 1;  // segments this launch runs
  const int seg = a.geo.n_seg > 1 ? 1 + r2 % nl : 0;
  const int pair = (r2 / nl) * 8 + xcd;
  if (pair >= a.n_seqs * a.H) return;
  scan_wg<K, V, Tin, Tout, NCH>(sms, a, pair, grp, seg);
}

// First launch of the chunk-parallel form (bf16 inputs, two slices per scan
// workgroup): the scan of every sequence's segment 0 (blocks [0, n_scan0))
// side by side with the maps of segments 1 .. n_seg - 2 (the remaining
// blocks), which need no state. Both kinds of workgroup have five waves and use
// one LDS layout (the summary's third and fourth V slices live in the q-tile
// buffers, which its workgroups do not otherwise use).
template <int K, int V, typename Tout>
__global__ __launch_bounds__(scan_threads<2>()) __attribute__((amdgpu_waves_per_eu(2, 2))) void seg0_kernel(
    ScanArgs<__bf16, Tout> a, int n_scan0) {
  GDN_SCAN_LDS(K, __bf16, 2)
  const int bid = blockIdx.x;
  if (bid < n_scan0) {
    constexpr int NG = V / 16 / 2;
    const int xcd = bid & 7, rest = bid >> 3;
    const int pair = (rest / NG) * 8 + xcd;
    if (pair >= a.n_seqs * a.H) return;
    scan_wg<K, V, __bf16, Tout, 2>(sms, a, pair, rest % NG, 0);
  } else {
    using S4 = ScanSmem<K, __bf16, 4>;
    static_assert(sizeof(lds_qt) >= 2 * sizeof(lds_v[0]), "two more V slices fit the q-tile buffers");
    typedef __bf16 VBuf[kChunk * 16];
    VBuf* v2 = reinterpret_cast<VBuf*>(&lds_qt[0][0]);
    S4 s4[4];
    s4[0] = S4{lds_k, lds_a, lds_v[0], lds_gx, nullptr, nullptr, nullptr, nullptr, nullptr, {nullptr, nullptr}, nullptr};
    s4[1] = S4{lds_k, lds_a, lds_v[1], lds_gx, nullptr, nullptr, nullptr, nullptr, nullptr, {nullptr, nullptr}, nullptr};
    s4[2] = S4{lds_k, lds_a, v2, lds_gx, nullptr, nullptr, nullptr, nullptr, nullptr, {nullptr, nullptr}, nullptr};
    s4[3] = S4{lds_k, lds_a, v2 + 2, lds_gx, nullptr, nullptr, nullptr, nullptr, nullptr, {nullptr, nullptr}, nullptr};
    constexpr int NGA = (V / 16 + K / 16) / 4;
    const int b2 = bid - n_scan0;  // n_scan0 is a multiple of 8: b2 keeps the XCD of bid
    const int xcd = b2 & 7, rest = b2 >> 3;
    const int grp = rest % NGA, r2 = rest / NGA;
    const int nm = a.geo.n_seg - 2;  // maps per sequence
    const int seg = 1 + r2 % nm;
    const int pair = (r2 / nm) * 8 + xcd;
    if (pair >= a.n_seqs * a.H) return;
    summary_wg<K, V, Tout>(s4, a, pair, grp, seg);
  }
}
#undef GDN_SCAN_LDS

// ---------------------------------------------------------------------------
// Host side: workspace layout and launch sequence.
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Segments per sequence for the chunk-parallel form (bf16 inputs), 1 where it
// is not taken. Its first launch runs every sequence's segment 0 (NG two-slice
// scan workgroups per pair) beside the maps of segments 1 .. n - 2 (NGA
// summary workgroups per pair and map); the second runs segments 1 .. n - 1
// (NG per pair and segment). n is the largest count for which both launches
// fit the compute units at once (at most kMaxSegments), taken if it is at
// least 3 (with 2, segment 1 would simply wait for segment 0).
constexpr int kSegCUs = 256;
static int segment_cap(int64_t pairs, int K, int V, bool in_f32, int n_cus = kSegCUs) {
  if (in_f32 || pairs <= 0) return 1;
  const int64_t p8 = (pairs + 7) / 8 * 8;
  const int64_t ng = V / 16 / 2, nga = (V / 16 + K / 16) / 4;
  int64_t n = std::min<int64_t>(kMaxSegments, n_cus / (p8 * ng) + 1);
  if (n_cus / p8 < ng) return 1;
  n = std::min<int64_t>(n, 2 + (n_cus / p8 - ng) / nga);
  return n >= 3 ? static_cast<int>(n) : 1;
}

// Lengths of the chunk-parallel form's segments for the longest sequence (nc
// chunks, n segments), from a cost model of the two launches in chain steps
// (measured on MI355X at B = 1, H = 16, K = V = 128: a step of segment 0 takes
// 1.57 us and its first step comes 0.75 us after a map's (it loads the initial
// state first), a step of a map 1.66, a step of a later segment 1.48, and a
// map fold 2.45 before the first step): the first launch lasts as long as the
// longer of segment 0 and a map, the second as long as its slowest segment,
// segment j (>= 1) folding j - 1 maps first. The last segment takes what
// remains, so shortening it (it folds the most maps) lengthens segment 0
// while the maps outlast it. For each L1 the cost is piecewise linear in L0;
// its breaks are the candidates.
static void segment_lengths(int nc, int n, int& L0_out, int& L1_out) {
  constexpr double ts = 1.57, t0 = 0.75, tm = 1.66, t1 = 1.48, F = 2.45;
  auto cost = [&](int L0, int L1) {
    const int last = nc - L0 - (n - 2) * L1;
    if (L0 < 1 || L1 < 1 || last < 1) return 1e300;
    const double first = std::max(t0 + L0 * ts, L1 * tm);
    const double later = std::max((n - 3) * F + L1 * t1, (n - 2) * F + last * t1);
    return first + later;
  };
  double best = 1e300;
  L1_out = (nc + n - 1) / n;
  L0_out = nc - (n - 1) * L1_out;
  for (int L1 = 1; (n - 2) * L1 + 2 <= nc; ++L1) {
    const int rest = nc - (n - 2) * L1;  // L0 + last
    const double a = (L1 * tm - t0) / ts;  // L0 where segment 0 starts to outlast the maps
    const double b = rest - ((n - 3) * F + L1 * t1 - (n - 2) * F) / t1;  // L0 where the last segment stops binding
    const int cand[6] = {static_cast<int>(a), static_cast<int>(a) + 1, static_cast<int>(b), static_cast<int>(b) + 1, 1,
                         rest - 1};
    for (int L0 : cand) {
      const double c = cost(L0, L1);
      if (c < best) {
        best = c;
        L0_out = L0;
        L1_out = L1;
      }
    }
  }
}

// The chunk-parallel form's segments for a call whose longest sequence has
// max_nc chunks ({1, 0, 0}: the single-pass scan).
SegPlan segment_plan(int64_t pairs, int K, int V, bool in_f32, int max_nc) {
  const int cap = segment_cap(pairs, K, V, in_f32);  // as the workspace was sized
  if (cap > 1 && max_nc >= 4 * 3) {
    const int n = std::min(cap, max_nc / 4);
    int L0 = 0, L1 = 0;
    segment_lengths(max_nc, n, L0, L1);
    if (n >= 3 && L0 >= 1) return SegPlan{n, L0, L1};
  }
  return SegPlan{1, 0, 0};
}

WsLayout workspace_layout(int64_t max_chunks, int n_seqs, int H, int K, int V, bool in_f32) {
  const size_t nch = static_cast<size_t>(max_chunks) * H;
  const int64_t pairs = static_cast<int64_t>(n_seqs) * H;
  WsLayout l{};
  l.max_segments = segment_cap(pairs, K, V, in_f32);
  size_t off = 0;
  l.af = off;
  off = align256(off + nch * kTileSetBytes);
  l.pf = off;
  off = align256(off + nch * kTileSetBytes);
  l.gx = off;
  off = align256(off + nch * 3 * kChunk * 4);
  l.info = off;
  off = align256(off + static_cast<size_t>(max_chunks) * 16);
  l.seq_chunk0 = off;
  off = align256(off + static_cast<size_t>(n_seqs + 1) * 4);
  const size_t sm = static_cast<size_t>(l.max_segments);
  l.seg_sum = off;
  if (sm > 1) off = align256(off + static_cast<size_t>(pairs) * (sm - 2) * (V + K) * K * 4);
  l.seg_state = off;
  if (sm > 1) off = align256(off + static_cast<size_t>(pairs) * V * K * 4);
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
  ws.seg_sum = reinterpret_cast<float*>(b + l.seg_sum);
  ws.seg_state = reinterpret_cast<float*>(b + l.seg_state);
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
    const int64_t prep_wgs = (a.n_chunks + 7) / 8 * 8 * a.H;  // at most INT32_MAX (checked by the caller)
    hipLaunchKernelGGL((prep_kernel<K, Tin>), dim3(static_cast<unsigned>(prep_wgs)), dim3(256), 0, a.stream,
                       static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), a.g, a.beta, a.H, a.scale,
                       a.T_eq, ncs_eq, static_cast<int>(a.total_tokens), static_cast<int>(a.n_chunks),
                       varlen ? a.ws.info : nullptr, a.ws);
  }
  if (a.events[1]) (void)hipEventRecord(a.events[1], a.stream);
  const int64_t pairs = static_cast<int64_t>(a.n_seqs) * a.H;
  const unsigned pair8 = static_cast<unsigned>((pairs + 7) / 8);
  ScanArgs<Tin, Tout> sa{static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), static_cast<const Tin*>(a.v),
                         static_cast<Tout*>(a.o), a.H, a.scale, a.n_seqs, a.T_eq, ncs_eq,
                         static_cast<int>(a.total_tokens), static_cast<int>(a.n_chunks), a.cu_seqlens, a.h0, a.ht,
                         a.pool, a.pool_slots, a.slots, SegGeom{1, 0, 0}, a.ws};
  // Chunk-parallel form where the scan would leave most compute units idle:
  // n segments per sequence, the first of L0 chunks, the others of L1, the
  // last of what remains. The first launch scans every segment 0 and forms the
  // maps of segments 1 .. n - 2; the second scans segments 1 .. n - 1 at once,
  // each from segment 0's final state carried through the maps of the
  // segments before its own.
  const SegPlan plan = segment_plan(pairs, K, V, !std::is_same<Tin, __bf16>::value, a.max_nc);
  if (plan.n_seg > 1) sa.geo = SegGeom{plan.n_seg, plan.L0, plan.L1};
  if constexpr (std::is_same<Tin, __bf16>::value) {
    if (sa.geo.n_seg > 1) {
      constexpr int NGA = (NSL + K / 16) / 4;
      const unsigned n_scan0 = 8 * (NSL / 2) * pair8;
      const unsigned n_sum = 8 * NGA * (sa.geo.n_seg - 2) * pair8;
      hipLaunchKernelGGL((seg0_kernel<K, V, Tout>), dim3(n_scan0 + n_sum), dim3(scan_threads<2>()), 0, a.stream, sa,
                         static_cast<int>(n_scan0));
      hipLaunchKernelGGL((scan_kernel<K, V, Tin, Tout, 2>), dim3(8 * (NSL / 2) * (sa.geo.n_seg - 1) * pair8),
                         dim3(scan_threads<2>()), 0, a.stream, sa);
      const hipError_t err = hipGetLastError();
      if (a.events[2]) (void)hipEventRecord(a.events[2], a.stream);
      return err;
    }
  }
  // Two chains per workgroup (sharing K, A' and the gates, on two SIMDs of a
  // CU) once one-chain workgroups would outnumber the compute units; bf16
  // inputs only (float32 operands would not leave room in LDS for the rest).
  bool two = false;
  if constexpr (std::is_same<Tin, __bf16>::value) {
    two = pairs * NSL > a.n_cus;
    if (two)
      hipLaunchKernelGGL((scan_kernel<K, V, Tin, Tout, 2>), dim3(8 * (NSL / 2) * pair8), dim3(scan_threads<2>()), 0,
                         a.stream, sa);
  }
  if (!two)
    hipLaunchKernelGGL((scan_kernel<K, V, Tin, Tout, 1>), dim3(8 * NSL * pair8), dim3(scan_threads<1>()), 0, a.stream,
                       sa);
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

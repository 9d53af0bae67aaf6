// Host-side interface between the C ABI (argument validation, workspace
// carving) and the kernel launchers. Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct DecodeArgs {
  const void *q, *k, *v;
  const float *g, *beta;  // g: [N, H] scalar log-gate, or [N, H, K] per key channel (kda)
  bool kda;
  float* pool;
  int64_t pool_slots;
  const int32_t* slots;
  void* o;
  int N, H, K, V;
  float scale;
  bool in_f32, out_f32;
  hipStream_t stream;
};

struct VerifyArgs {
  const void *q, *k, *v;
  const float *g, *beta;
  float* pool;
  int64_t pool_slots;
  const int32_t* slots;  // [N, cols]
  int cols;
  const int32_t* accepted;  // [N]
  void* o;
  int N, T, H, K, V;
  float scale;
  bool in_f32, out_f32;
  hipStream_t stream;
};

struct PrologueArgs {
  const void* x;            // [N, 3 H D] bf16
  const float* conv_w;      // [3, 4, H D]
  const float* conv_bias;   // [3 H D] or null
  void* conv_state;         // [pool_slots, 3 H D, 3] bf16
  int64_t pool_slots;
  const int32_t* slots;     // [N], or [N, cols] (verify: T tokens per request)
  int cols;                 // verify: slot columns
  const int32_t* accepted;  // verify: [N]
  const float* beta_raw;    // [N T, H]
  float *q, *k, *v, *beta;  // [N T, H, D] x 3, [N T, H]
  int N, T, H, D;
  hipStream_t stream;
};

struct LayerArgs {
  const void* x;            // [N, 3 H D] bf16
  const float* conv_w;      // [3, 4, H D]
  const float* conv_bias;   // [3 H D] or null
  void* conv_state;         // [conv_slots, 3 H D, 3] bf16
  int64_t conv_slots;
  const int32_t* slots;     // [N]
  const float* beta_raw;    // [N, H]
  const float* g;           // [N, H] or, kda, [N, H, D] log-decays
  bool kda;
  float* pool;              // [pool_slots, H, D, D]
  int64_t pool_slots;
  const void* gate;         // [N, H D] bf16 (with norm_w)
  const float* norm_w;      // [D], or null: the raw output
  float eps;
  void* out;                // [N, H, D]
  bool out_f32;
  int N, H, D;
  float scale;
  hipStream_t stream;
};

struct RmsNormArgs {
  const float* o;       // [N, H, D]
  const void* gate;     // [N, H D] bf16
  const float* norm_w;  // [D]
  float eps;
  void* out;            // [N, H, D]
  bool out_f32;
  int N, H, D;
  hipStream_t stream;
};

struct KdaChunkArgs {
  const void *q, *k, *v;  // [Ttot, H, K] / [Ttot, H, V]
  const float* g;         // [Ttot, H, K] per-channel log-decays
  const float* beta;      // [Ttot, H]
  void* o;                // [Ttot, H, V]
  int n_seqs;
  int64_t total_tokens;
  int H, K, V;
  float scale;
  bool in_f32, out_f32;
  const int32_t* cu_seqlens;  // device, or null for equal lengths
  int64_t n_chunks;           // total chunks over all sequences
  int T_eq;                   // equal-length mode: tokens per sequence
  const float* h0;  // [n_seqs, H, V, K] or null
  float* ht;        // [n_seqs, H, V, K] or null
  float* pool;      // [pool_slots, H, V, K] or null (then h0 / ht)
  int64_t pool_slots;
  const int32_t* slots;  // [n_seqs]
  void* ws;              // kda_workspace_bytes(...) bytes
  hipStream_t stream;
  hipEvent_t events[3];  // optional: before prep, after prep, after the scan
};
size_t kda_workspace_bytes(int64_t max_chunks, int n_seqs, int H, int K);
hipError_t launch_chunk_schedule(const int32_t* cu, int n_seqs, int total_tokens, int cap, int* seq_chunk0,
                                 int4* info, hipStream_t stream);

struct GateArgs {
  const void* f_a;      // [N, 128] bf16
  const void* f_b;      // [H * K, 128] bf16
  const float* a_log;   // [H]
  const float* dt_bias; // [H * K]
  float lower_bound;
  int mode;             // reduction order of the projection: 0, 1 or 2
  float* g;             // [N, H, K] log-decays
  void* raw_out;        // [N, H, K] bf16 projection, or null
  int N, H, K;
  hipStream_t stream;
};

struct Fp8Args {
  const float* x;     // [n_groups * group] float32
  void* codes;        // [n_groups * group] uint8 (E4M3)
  float* scales;      // [n_groups]
  int64_t n_groups;
  int group;          // 64 or 128
  hipStream_t stream;
};

// Chunk intermediates written by the prep kernel and read by the scan kernel.
// A fragment is stored as planes of [64 lanes][16 bytes] (see Prec in
// gdn_common.h: two planes for a computed operand). "ch" = chunk * H + head.
//   af  [ch][6 tiles][2 planes]      A' = A diag(beta) as A operands: the
//        nonzero (output row tile rt, token block ks) tiles (0,0) (1,0) (2,0)
//        (2,1) (3,0) (3,1) in that order
//   pf  [ch][6 tiles][2 planes]      P = s (Q K^T) * E * M, the same way
//   gx  [ch][3][64] f32              g (chunk-local inclusive cumulative sum of
//        the log-gate; rows past the chunk end repeat g_last), e^g, e^{g_last - g}
//   info [chunk] int4 {seq, first token, rows, 0} and seq_chunk0 [n_seqs + 1]:
//        the chunk schedule of a packed (varlen) call
//   seg_sum [pair][n_seg - 2][(V + K) K] f32  chunk-parallel form: for segments
//        1 .. n_seg - 2, the affine map of the state h -> M h + c: c^T rows
//        [v][key] (float32), then M as split bf16 A-operand fragments (MapFrag)
//   seg_state [pair][V][K] f32                 segment 0's final state, where
//        every later segment of the pair starts
struct ChunkWs {
  uint8_t* af;
  uint8_t* pf;
  float* gx;
  int4* info;
  int* seq_chunk0;
  float* seg_sum;
  float* seg_state;
};

struct ChunkArgs {
  const void *q, *k, *v;
  const float *g, *beta;
  void* o;
  int n_seqs;
  int64_t total_tokens;
  int H, K, V;
  float scale;
  bool in_f32, out_f32;
  const int32_t* cu_seqlens;  // device, or null for equal lengths
  int64_t n_chunks;           // total chunks over all sequences
  int max_nc;                 // chunks of the longest sequence
  int T_eq;                   // equal-length mode: tokens per sequence
  const float* h0;
  float* ht;
  float* pool;
  int64_t pool_slots;
  const int32_t* slots;
  ChunkWs ws;
  int n_cus;  // compute units of the current device (sizes the scan's workgroups)
  hipStream_t stream;
  hipEvent_t events[3];  // optional: recorded before prep, after prep, after scan
};

// Workspace layout for a call with at most max_chunks chunks.
struct WsLayout {
  size_t af, pf, gx, info, seq_chunk0, seg_sum, seg_state, total;
  int max_segments;  // segments per sequence the chunk-parallel form may use (1: not used)
};
WsLayout workspace_layout(int64_t max_chunks, int n_seqs, int H, int K, int V, bool in_f32);
// Segments of the chunk-parallel form: n_seg per sequence (1: single pass),
// segment 0 of L0 chunks, segments 1 .. n_seg - 2 of L1, the last the rest.
struct SegPlan {
  int n_seg, L0, L1;
};
SegPlan segment_plan(int64_t pairs, int K, int V, bool in_f32, int max_nc);
ChunkWs carve_workspace(const WsLayout& l, void* base);

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_verify(const VerifyArgs& a);
hipError_t launch_fp8_quant(const Fp8Args& a);
hipError_t launch_decode_prologue(const PrologueArgs& a);
hipError_t launch_decode_prologue_verify(const PrologueArgs& a);
hipError_t launch_gated_rmsnorm(const RmsNormArgs& a);
hipError_t launch_decode_layer(const LayerArgs& a);
hipError_t launch_chunk_fwd_kda(const KdaChunkArgs& a);
hipError_t launch_chunk_fwd(const ChunkArgs& a);
hipError_t launch_kda_gate(const GateArgs& a);

}  // namespace gdn

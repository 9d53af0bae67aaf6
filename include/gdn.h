/*
 * gdn.h - C ABI of the MI355X (gfx950) gated delta rule library.
 *
 * Two operations:
 *
 *  gdn_chunk_fwd       the chunked forward pass of the gated delta rule
 *                      (GatedDeltaNet): recompute_w_u, then chunk_fwd_h, then
 *                      chunk_fwd_o over chunks of 64 tokens, as the WarpDrive
 *                      page describes them (kernels 5, 3, 4 and its "Pipeline"
 *                      paragraph);
 *  gdn_recurrent_step  one token of the same rule per request over a
 *                      slot-indexed state pool, as the vLLM KdaSplit page's
 *                      decode kernel runs it (class docstring and method
 *                      update), with one scalar decay per token and head.
 *
 * Per sequence and head, with q_t, k_t in R^K, v_t in R^V, beta_t in (0,1), the
 * raw log-gate a_t <= 0 and the query scale s, both compute
 *
 *      S <- exp(a_t) S;  S <- S + beta_t (v_t - S k_t) k_t^T;  o_t = S (s q_t)
 *
 * where S is the V x K state (rows = value channels, columns = key channels).
 *
 * Conventions shared by every entry point:
 *  - Pointers are device pointers owned by the caller unless stated otherwise.
 *    The library allocates nothing and keeps no state between calls (the one
 *    exception, gdn_chunk_fwd_noalloc's device array, holds no state either:
 *    its contents on entry are ignored).
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *    Calls return without waiting for the GPU.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is launched and the status says why. GDN_EHIP reports a
 *    launch failure from the HIP runtime.
 *  - Layouts are dense row-major with the last index contiguous. Tensors of the
 *    input dtype (q, k, v) and the output o must be 16-byte aligned; float
 *    arrays 4-byte aligned.
 *  - Supported head sizes: K in {64, 128}, V in {64, 128}.
 *  - States (h0, ht, pools) are float32 [.., H, V, K].
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_EINVAL = -1,       /* bad pointer, size, alignment, or inconsistent lengths */
  GDN_EUNSUPPORTED = -2, /* K or V not in {64, 128}, or an unknown dtype */
  GDN_EWORKSPACE = -3,   /* workspace NULL or smaller than required */
  GDN_EHIP = -4          /* the HIP runtime reported an error at launch */
} gdn_status;

typedef enum gdn_dtype {
  GDN_BF16 = 0, /* bfloat16 */
  GDN_F32 = 1   /* float32 */
} gdn_dtype;

/*
 * Bytes of device workspace gdn_chunk_fwd needs for a call with these sizes
 * (an upper bound valid for every split of total_tokens into n_seqs
 * sequences). Returns 0 for invalid sizes. The workspace holds the chunk
 * intermediates of recompute_w_u in the form the scan consumes (A' = A diag(beta)
 * of the WY matrix A, from which u - w h = A'(V - diag(e^g) K h) follows), the
 * masked intra-chunk scores, the chunk-local gate sums, the chunk schedule
 * and, for bfloat16 inputs with few (sequence, head) pairs, the chunk-parallel
 * form's per-segment state maps and initial states.
 */
size_t gdn_chunk_fwd_workspace_bytes(int n_seqs, int64_t total_tokens, int H, int K, int V,
                                     gdn_dtype in_dtype);

/*
 * Where gdn_chunk_fwd leaves its intermediates in the workspace for a call
 * with these sizes (max_len: tokens of the longest sequence), so that they can
 * be inspected after the call returns and before the workspace is reused:
 * recompute_w_u's outputs and, in the chunk-parallel form, the segment states
 * and maps of chunk_fwd_h (WarpDrive page, kernels 5 and 3, "Pipeline").
 * Host only, no device access; GDN_EINVAL for invalid sizes or null outputs,
 * GDN_EUNSUPPORTED for head sizes or dtypes gdn_chunk_fwd does not take.
 *  plan[3]     segments per sequence n (1: every sequence scanned in one pass),
 *              chunks of segment 0, chunks of each of segments 1 .. n - 2 (the
 *              last segment has what remains)
 *  offsets[5]  byte offsets from the workspace base of:
 *   [0] A' = A diag(beta): per (chunk, head), ch = chunk * H + head (chunks
 *       numbered sequence by sequence), 6 tiles (row tile rt, token block ks) =
 *       (0,0) (1,0) (2,0) (2,1) (3,0) (3,1), each two planes of 64 lanes x 16
 *       bytes; lane l = 16 g + c holds row 16 rt + c at the token columns
 *       32 ks + kappa(g, e), e = 0..7, kappa(g, e) = 4 g + e for e < 4 and
 *       16 + 4 g + (e - 4) otherwise; bfloat16 inputs: plane 0 the bfloat16
 *       high parts, plane 1 the low parts (value = high + low); float32 inputs:
 *       plane 0 values e = 0..3, plane 1 values e = 4..7, as float32
 *   [1] P = s (Q K^T) * E * M, the same way
 *   [2] the gate vectors, per ch 3 x 64 float32: g (chunk-local inclusive sum;
 *       rows past a chunk's end repeat its last), e^g, e^{g_last - g}
 *   [3] the maps of segments 1 .. n - 2 (n >= 3), per pair = sequence * H +
 *       head and segment, (V + K) K float32 words: c^T as rows [v][key], then
 *       M (h_out = M h_in + c for the [K, V] state) as K / 32 x K / 16
 *       fragments (key block kb, state tile t) of two bfloat16 planes (high,
 *       low) of 64 lanes x 16 bytes, lane 16 g + c holding row
 *       32 (t / 2) + 8 (c / 4) + 4 (t % 2) + c % 4 of M at columns
 *       32 kb + 8 g + e, e = 0..7
 *   [4] segment 0's final state per pair, [V][K] float32 (n >= 3)
 */
gdn_status gdn_chunk_fwd_plan(int n_seqs, int64_t total_tokens, int64_t max_len, int H, int K, int V,
                              gdn_dtype in_dtype, int32_t* plan, int64_t* offsets);

/*
 * Chunked forward pass over n_seqs sequences packed into one token stream.
 *
 *  q, k        [total_tokens, H, K] in_dtype   queries, keys (the library does
 *                                              not normalise them)
 *  v           [total_tokens, H, V] in_dtype   values
 *  g           [total_tokens, H] float32       raw per-token log-gate a_t (<= 0),
 *                                              NOT cumulated: the library takes the
 *                                              inclusive sum within each chunk
 *  beta        [total_tokens, H] float32       write strengths
 *  o           [total_tokens, H, V] out_dtype  output (written; rows are tokens)
 *  scale       multiplies q only
 *  cu_seqlens  device int32 [n_seqs + 1] sequence offsets, or NULL: then the
 *              n_seqs sequences have equal length total_tokens / n_seqs
 *  cu_seqlens_host  host copy of cu_seqlens (sizes the launch grid); NULL iff
 *              cu_seqlens is NULL. Must start at 0, never decrease and end at
 *              total_tokens.
 *  h0, ht      float32 [n_seqs, H, V, K]: initial state (NULL = zeros) and final
 *              state (NULL = not stored). They may alias (in-place update).
 *  state_pool, pool_slots, state_slots
 *              alternative to h0/ht: float32 pool [pool_slots, H, V, K] and
 *              device int32 state_slots[n_seqs]. Sequence i reads its initial
 *              state from and writes its final state to pool[state_slots[i]] in
 *              place; a slot <= 0 means a zero initial state and no write, and a
 *              slot >= pool_slots is treated the same way. Active slots must be
 *              distinct. When state_pool is given, h0 and ht must be NULL.
 *  workspace   device scratch of at least gdn_chunk_fwd_workspace_bytes(...)
 *              bytes, 256-byte aligned; contents on entry are ignored.
 *
 * Size limits (GDN_EINVAL beyond them): H in [1, 65535], total_tokens below
 * 2^31 - 128, n_seqs H at most 2^28, and (total_tokens / 64 + n_seqs) H, the
 * (chunk, head) count the call is sized for, below 2^31 - 8 H.
 *
 * Chunks of 64 tokens start at every sequence start; a sequence's last chunk
 * may be shorter. An empty sequence passes its initial state to ht unchanged.
 * The result is deterministic: identical calls give identical bits, and o in
 * bfloat16 equals round-to-nearest-even of the float32 result of the same call.
 */
gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, void* o, int n_seqs, int64_t total_tokens, int H,
                         int K, int V, float scale, gdn_dtype in_dtype, gdn_dtype out_dtype,
                         const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                         const float* h0, float* ht, float* state_pool, int64_t pool_slots,
                         const int32_t* state_slots, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Diagnostic variant of gdn_chunk_fwd for measurement: same arguments, same
 * results, and in addition it records three caller-created HIP events
 * (hipEvent_t, passed as void*) on `stream`: events[0] before the first kernel,
 * events[1] after the prep kernel (recompute_w_u: gate sums, K K^T, triangular
 * solve, A' and the masked intra-chunk scores), events[2] after chunk_fwd_h
 * fused with chunk_fwd_o (the scan kernel, preceded in the chunk-parallel form
 * by the segment summary and combine kernels). hipEventElapsedTime of
 * consecutive events then gives each part's duration on that stream.
 * `events` must point to three valid events; GDN_EINVAL otherwise.
 */
gdn_status gdn_chunk_fwd_profiled(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, void* o, int n_seqs, int64_t total_tokens,
                                  int H, int K, int V, float scale, gdn_dtype in_dtype,
                                  gdn_dtype out_dtype, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_host, const float* h0, float* ht,
                                  float* state_pool, int64_t pool_slots,
                                  const int32_t* state_slots, void* workspace,
                                  size_t workspace_bytes, void* stream, void* const* events);

/*
 * Bytes of the device array that backs gdn_chunk_fwd_noalloc's workspace: the
 * largest gdn_chunk_fwd_workspace_bytes(...) that entry point accepts (64 MiB;
 * e.g. B=1, H=16, T=4096, K=V=128 in bfloat16 needs about 33 MB).
 */
#define GDN_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments (without workspace and workspace_bytes), same launches, same
 * results bit for bit; the workspace is a file-scope device array of the
 * library, GDN_NOALLOC_WORKSPACE_BYTES bytes, of which each GPU the library runs
 * on holds its own copy until the process ends. Nothing is allocated and the
 * array's contents on entry are ignored (every call writes what it reads).
 *
 * The device is the current HIP device, which must be the stream's. Calls on
 * one GPU share that GPU's array: two calls whose work overlaps on the GPU (on
 * different streams, or from different host threads without ordering) race and
 * give undefined results; calls in one stream are ordered and safe.
 *
 * Returns GDN_EWORKSPACE, without launching, when
 * gdn_chunk_fwd_workspace_bytes(n_seqs, total_tokens, H, K, V, in_dtype) exceeds
 * GDN_NOALLOC_WORKSPACE_BYTES; GDN_EHIP if the array's device address cannot
 * be obtained or a launch fails; otherwise every status as gdn_chunk_fwd.
 */
gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, void* o, int n_seqs, int64_t total_tokens, int H,
                                 int K, int V, float scale, gdn_dtype in_dtype, gdn_dtype out_dtype,
                                 const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                 const float* h0, float* ht, float* state_pool, int64_t pool_slots,
                                 const int32_t* state_slots, void* stream);

/*
 * One decode step for N requests over a slot-indexed state pool (the vLLM
 * KdaSplit page: state [slot, head, value, key], slots <= 0 are padding).
 *
 *  q, k        [N, H, K] in_dtype;  v [N, H, V] in_dtype
 *  g, beta     [N, H] float32 raw log-gate a (<= 0) and write strength
 *  state_pool  float32 [pool_slots, H, V, K], updated in place for active rows
 *  slots       device int32 [N]; slot <= 0 marks padding: its o rows are +0 and
 *              the pool is not touched. A slot >= pool_slots is treated as
 *              padding. Active slots must be distinct.
 *  o           [N, H, V] out_dtype
 *
 * Per active row b and head h: S = pool[slots[b], h]; S <- exp(a) S;
 * S <- S + beta (v - S k) k^T; o = S (scale q); the updated S is stored back.
 *
 * Returns GDN_EUNSUPPORTED for K or V outside {64, 128} or an unknown dtype;
 * GDN_EINVAL for N < 0, H outside [1, 65535], N * H * V / 16 > INT32_MAX (one
 * workgroup per 16 state rows), a NULL pointer, pool_slots <= 0 or a misaligned
 * pointer (pool 16 bytes, g / beta / slots 4 bytes, q / k / v / o their element
 * size); GDN_OK without launching for N == 0; GDN_EHIP if the launch fails.
 */
gdn_status gdn_recurrent_step(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, float* state_pool, int64_t pool_slots,
                              const int32_t* slots, void* o, int N, int H, int K, int V,
                              float scale, gdn_dtype in_dtype, gdn_dtype out_dtype, void* stream);

/*
 * gdn_recurrent_step with a decay per key channel (the vLLM KdaSplit page, method
 * update: every state element of key column e is multiplied by that column's
 * decay before the delta-rule write).
 *
 *  g           float32 [N, H, K], 16-byte aligned: the per-channel log-decay
 *              (<= 0); every other argument as in gdn_recurrent_step
 *
 * Per active row b and head h: S = pool[slots[b], h]; S <- S diag(exp(g[b, h]));
 * S <- S + beta (v - S k) k^T; o = S (scale q); the updated S is stored back.
 * Status codes as gdn_recurrent_step (g must be 16-byte aligned).
 */
gdn_status gdn_recurrent_step_kda(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, float* state_pool, int64_t pool_slots,
                                  const int32_t* slots, void* o, int N, int H, int K, int V,
                                  float scale, gdn_dtype in_dtype, gdn_dtype out_dtype,
                                  void* stream);

/*
 * Speculative-verify decode: T tokens per request (the vLLM KdaSplit page, class
 * docstring, ``tokens`` q > 1, with its spec-cache semantics).
 *
 *  q, k        [N * T, H, K] in_dtype, rows b * T + t;  v [N * T, H, V] in_dtype
 *  g, beta     [N * T, H] float32 raw log-gate a (<= 0) and write strength
 *  state_pool  float32 [pool_slots, H, V, K]
 *  slots       device int32 [N, slot_cols] (row-major), slot_cols >= T
 *  accepted    device int32 [N]
 *  o           [N * T, H, V] out_dtype
 *
 * Request b starts from pool[slots[b, accepted[b] - 1]] and runs its T tokens in
 * order, each one step of gdn_recurrent_step (decay, delta-rule write, output from
 * the updated state); the state after token t is stored to pool[slots[b, t]] if
 * that slot is in [1, pool_slots). A request whose source slot is outside
 * [1, pool_slots), or whose accepted count is outside [1, slot_cols], is padding:
 * its T output rows are +0 and nothing is written. The source is read before any
 * write of the request (so slots[b, accepted - 1] may be rewritten by it);
 * positive slots written by different requests, and their sources, must be
 * distinct.
 *
 * Returns GDN_EUNSUPPORTED for K or V outside {64, 128} or an unknown dtype;
 * GDN_EINVAL for N < 0, T outside [1, 8], slot_cols < T, H outside [1, 65535],
 * sizes whose grid would not fit, a NULL pointer, pool_slots <= 0 or a
 * misaligned pointer; GDN_OK without launching for N == 0; GDN_EHIP if the launch
 * fails.
 */
gdn_status gdn_recurrent_verify(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, float* state_pool, int64_t pool_slots,
                                const int32_t* slots, int slot_cols, const int32_t* accepted, void* o,
                                int N, int T, int H, int K, int V, float scale, gdn_dtype in_dtype,
                                gdn_dtype out_dtype, void* stream);

/*
 * Per-key-channel decays of the KDA decode layer from its low-rank gate
 * projection (the vLLM KdaSplit page, method gate_warp and its multicast): for
 * token t, head h and key channel f,
 *
 *   raw  = sum over c < 128 of f_a[t, c] * f_b[h K + f, c]     (float32)
 *   g    = lower_bound * sigmoid(exp(a_log[h]) * (bf16(raw) + dt_bias[h K + f]))
 *
 * with bf16() round to nearest even; the decay is exp(g), so g is the log-decay
 * gdn_recurrent_step_kda and gdn_chunk_fwd_kda take.
 *
 *  f_a       bf16 [N, 128]   the gate's activations (rank 128), 16-byte aligned
 *  f_b       bf16 [H * K, 128] the projection weight, 16-byte aligned
 *  a_log     float32 [H];  dt_bias float32 [H * K]
 *  lower_bound  finite float (the log-decay at gate 1; <= 0 for decays <= 1)
 *  mode      float32 reduction order of raw, as the page names them:
 *            0 = one chain over the 128 columns; 1 = four chains of 32 columns,
 *            summed 0 + (((c0 + c1) + c2) + c3); 2 = sixteen partials of 8
 *            columns summed in a butterfly (p[i] += p[i + 2^s], s = 3, 2, 1, 0).
 *            Each is a fixed sequence of IEEE float32 fused multiply-adds (in
 *            column order) and adds, so bf16(raw) is reproducible bit for bit.
 *  g         float32 [N, H, K] (output)
 *  raw_g     bf16 [N, H, K] (output: bf16(raw)), or NULL
 *
 * Returns GDN_EUNSUPPORTED for K outside {64, 128}; GDN_EINVAL for a mode
 * outside {0, 1, 2}, N < 0, H outside [1, 65535], ceil(N / 8) * 8 ceil(H / 8)
 * above 2^31 - 1, a non-finite lower_bound, a NULL or misaligned pointer (raw_g
 * may be NULL); GDN_OK without launching for N == 0; GDN_EHIP if the launch
 * fails.
 */
gdn_status gdn_kda_gate(const void* f_a, const void* f_b, const float* a_log, const float* dt_bias,
                        float lower_bound, int mode, float* g, void* raw_g, int N, int H, int K,
                        void* stream);

/*
 * FP8 group quantisation (the WarpDrive page, kernel 1, fp8_quant).
 *
 *  x       float32 [rows, cols], row-major, 16-byte aligned; finite values
 *  codes   uint8 [rows, cols] (E4M3 "fn": sign, 4 exponent bits with bias 7,
 *          3 mantissa bits, largest finite 448), 4-byte aligned
 *  scales  float32 [rows, cols / group]
 *  group   64 or 128 consecutive elements of a row
 *
 * Per group: scale = absmax / 448 (float32); each element is divided by scale
 * (float32), clamped to [-448, 448] and rounded to the nearest E4M3 value, ties to
 * even. A group whose absmax is 0 gets scale 0 and codes 0. x * scale of the
 * decoded codes approximates x to half an E4M3 unit in the last place.
 *
 * Returns GDN_EUNSUPPORTED for a group other than 64 or 128; GDN_EINVAL for
 * negative sizes, cols not a multiple of group, sizes whose grid would not fit,
 * a NULL or misaligned pointer; GDN_OK without launching when there is nothing
 * to do; GDN_EHIP if the launch fails.
 */
gdn_status gdn_fp8_quant(const float* x, void* codes, float* scales, int64_t rows, int64_t cols,
                         int group, void* stream);

/*
 * Front operations of a decode layer (vLLM KdaSplit page, kernel body: the
 * convolution, activation and normalisation steps before the recurrent update),
 * one token per request, for heads of D = K = V channels.
 *
 *  x           bf16 [N, 3 H D]: the token's projected q, k, v sections, each
 *              [H, D] (channel h D + c of a section)
 *  conv_w      float32 [3, 4, H D]: per section, tap (oldest first) and channel
 *  conv_bias   float32 [3 H D], or NULL for none
 *  conv_state  bf16 [pool_slots, 3 H D, 3]: the slot's previous three inputs per
 *              channel, oldest first; updated in place for active rows to its
 *              last two entries followed by x
 *  slots       device int32 [N]; slot <= 0 or >= pool_slots marks padding: its
 *              q, k, v rows and beta are +0 and conv_state is not touched.
 *              Active slots must be distinct.
 *  beta_raw    float32 [N, H]
 *  q, k, v     float32 [N, H, D] (outputs; the layout the decode step reads)
 *  beta        float32 [N, H] (output)
 *
 * Per channel: y = SiLU(bias + sum over the 4 taps of w * input), with the
 * window (conv_state[slot, ch, 0..2], x); then each head's q and k are divided by
 * sqrt(sum of squares + 1e-6) and beta = sigmoid(beta_raw). The query scale is
 * not applied here (the decode step takes it).
 *
 * Alignment: x, conv_state, beta_raw, beta and slots 4 bytes; conv_w, conv_bias,
 * q, k and v 8 bytes (each lane moves two adjacent channels).
 *
 * Returns GDN_EUNSUPPORTED for D outside {64, 128}; GDN_EINVAL for N < 0, H
 * outside [1, 65535], N H above 2^31 - 1, a NULL pointer (other than conv_bias),
 * pool_slots <= 0 or a misaligned pointer; GDN_OK without launching for N == 0;
 * GDN_EHIP if the launch fails.
 */
gdn_status gdn_decode_prologue(const void* x, const float* conv_w, const float* conv_bias,
                               void* conv_state, int64_t pool_slots, const int32_t* slots,
                               const float* beta_raw, float* q, float* k, float* v, float* beta,
                               int N, int H, int D, void* stream);

/*
 * Front operations of a decode layer for T tokens per request (speculative
 * verify: the vLLM KdaSplit page, class docstring, ``tokens`` q > 1, and the
 * kernel body's multi-token conv window and rewrite), heads of D = K = V
 * channels. Rows of x, beta_raw and the outputs are b * T + t.
 *
 *  x           bf16 [N * T, 3 H D]: the tokens' projected q, k, v sections
 *  conv_w      float32 [3, 4, H D];  conv_bias float32 [3 H D] or NULL
 *  conv_state  bf16 [pool_slots, 3 H D, T + 2]: request b's conv page is
 *              slot[b, 0]; its columns a - 1, a, a + 1 (a = accepted[b]) are
 *              the three inputs before the request's first token. Updated in
 *              place for active requests to (column a, column a + 1, x_0, ...,
 *              x_{T-1}).
 *  slots       device int32 [N, slot_cols] (row-major), slot_cols >= T; the
 *              recurrent state's source is slot[b, a - 1] (as in
 *              gdn_recurrent_verify)
 *  accepted    device int32 [N]
 *  beta_raw    float32 [N * T, H]
 *  q, k, v     float32 [N * T, H, D] (outputs);  beta float32 [N * T, H]
 *
 * Token t's channel takes y = SiLU(bias + sum over the 4 taps of w * window)
 * with the window (page column a - 1 + t .. , then the inputs) at positions
 * t .. t + 3 of (three page columns, x_0 .. x_{T-1}); then each head's q and k
 * are divided by sqrt(sum of squares + 1e-6) and beta = sigmoid(beta_raw).
 * A request whose accepted count is outside [1, T], whose source slot is <= 0,
 * or whose conv slot is outside [1, pool_slots) is padding: its rows are +0 and
 * its conv page is not touched. Active conv slots must be distinct.
 *
 * Alignment: x, slots, accepted, beta_raw and beta 4 bytes; conv_state 2 bytes;
 * conv_w, conv_bias, q, k and v 8 bytes.
 *
 * Returns GDN_EUNSUPPORTED for D outside {64, 128}; GDN_EINVAL for N < 0, T
 * outside [1, 8], slot_cols < T, H outside [1, 65535], sizes whose grid would not
 * fit, a NULL pointer (other than conv_bias), pool_slots <= 0 or a misaligned
 * pointer; GDN_OK without launching for N == 0; GDN_EHIP if the launch fails.
 */
gdn_status gdn_decode_prologue_verify(const void* x, const float* conv_w, const float* conv_bias,
                                      void* conv_state, int64_t pool_slots, const int32_t* slots,
                                      int slot_cols, const int32_t* accepted, const float* beta_raw,
                                      float* q, float* k, float* v, float* beta, int N, int T, int H,
                                      int D, void* stream);

/*
 * Gated RMSNorm of each head's decode output (vLLM KdaSplit page, kernel body:
 * the output normalisation after the recurrent update).
 *
 *  o       float32 [N, H, D] (the decode step's output in float32)
 *  gate    bf16 [N, H D] (raw gate; sigmoid is applied here)
 *  norm_w  float32 [D], shared by the heads
 *  out     [N, H, D] in out_dtype (bf16 or float32); may not alias o
 *
 * out = o * rsqrt(mean over the head's D channels of o^2 + eps) * norm_w[c] *
 * sigmoid(gate), in float32.
 *
 * Alignment: o and norm_w 8 bytes; gate 4 bytes; out 4 bytes (bf16) or 8 bytes
 * (float32).
 *
 * Returns GDN_EUNSUPPORTED for D outside {64, 128} or an unknown dtype;
 * GDN_EINVAL for N < 0, H outside [1, 65535], N H above 2^31 - 1, eps < 0 or
 * NaN, a NULL or misaligned pointer; GDN_OK without launching for N == 0;
 * GDN_EHIP if the launch fails.
 */
gdn_status gdn_gated_rmsnorm(const float* o, const void* gate, const float* norm_w, float eps,
                             void* out, int N, int H, int D, gdn_dtype out_dtype, void* stream);

/*
 * The decode layer in one launch, one token per request (the vLLM KdaSplit page,
 * kernel body: convolution, activation and normalisation steps, the recurrent
 * update, the output norm), for heads of D = K = V channels: the steps of
 * gdn_decode_prologue, then gdn_recurrent_step (g_per_channel = 0: g [N, H]) or
 * gdn_recurrent_step_kda (g_per_channel != 0: g [N, H, D], 16-byte aligned) on
 * its q, k, v and beta, then gdn_gated_rmsnorm (when norm_w is not NULL; else
 * out is the raw update output). Every argument as in those entry points;
 * the conv-state pool has conv_slots slots and the state pool pool_slots, both
 * indexed by slots[b]; a slot <= 0 or outside either pool is padding (out row
 * +0, neither pool touched). Active slots must be distinct.
 *
 *  x           bf16 [N, 3 H D];  conv_w float32 [3, 4, H D];  conv_bias [3 H D] or NULL
 *  conv_state  bf16 [conv_slots, 3 H D, 3] (in place)
 *  beta_raw    float32 [N, H]
 *  state_pool  float32 [pool_slots, H, D, D] (in place)
 *  gate        bf16 [N, H D] (with norm_w);  norm_w float32 [D] or NULL;  eps >= 0
 *  out         [N, H, D] out_dtype
 *  scale       multiplies the normalised q
 *
 * Returns GDN_EUNSUPPORTED for D outside {64, 128} or an unknown dtype;
 * GDN_EINVAL for N < 0, H outside [1, 65535], N H above 2^31 - 1, a negative or
 * NaN eps with norm_w, a NULL pointer (other than conv_bias, norm_w and then
 * gate), a pool size <= 0 or a misaligned pointer; GDN_OK without launching for
 * N == 0; GDN_EHIP if the launch fails.
 */
gdn_status gdn_decode_layer(const void* x, const float* conv_w, const float* conv_bias, void* conv_state,
                            int64_t conv_slots, const int32_t* slots, const float* beta_raw,
                            const float* g, int g_per_channel, float* state_pool, int64_t pool_slots,
                            const void* gate, const float* norm_w, float eps, void* out,
                            gdn_dtype out_dtype, int N, int H, int D, float scale, void* stream);

/*
 * Bytes of device workspace gdn_chunk_fwd_kda needs (an upper bound valid for
 * every split of total_tokens into n_seqs sequences): per (chunk of 64 tokens,
 * head) (2 * 64 * 64 + 3 * 64 * K + K) float32 of chunk operands, then the chunk
 * schedule of a packed call. Returns 0 for invalid sizes.
 */
size_t gdn_chunk_fwd_kda_workspace_bytes(int n_seqs, int64_t total_tokens, int H, int K);

/*
 * Chunked forward pass of the delta rule with a decay per key channel (vLLM
 * KdaSplit page, method `update`: each key column of the state is multiplied by
 * its own decay before the delta-rule write; here in the chunk form, chunks of 64
 * tokens) over n_seqs sequences packed into one token stream. Arguments as in
 * gdn_chunk_fwd, except:
 *
 *  g         float32 [total_tokens, H, K], 16-byte aligned: per-token,
 *            per-key-channel log-decays (<= 0; -inf, a channel that forgets
 *            everything, is accepted), raw (the library sums them within each
 *            chunk)
 *  q, k      16-byte aligned (read four channels at a time); v, o by their
 *            element size; beta, states, pool and slots 4 bytes
 *  workspace at least gdn_chunk_fwd_kda_workspace_bytes(n_seqs, total_tokens,
 *            H, K) bytes, 256-byte aligned
 *  V         a multiple of 16 in [16, 256]
 *
 * Per token: S <- S diag(exp(g_t)); delta = beta_t (v_t - S k_t);
 * S <- S + delta k_t^T; o_t = S (scale q_t). cu_seqlens (device) and
 * cu_seqlens_host (host) give the sequence offsets, or are both NULL for
 * n_seqs sequences of total_tokens / n_seqs tokens. States: h0 / ht float32
 * [n_seqs, H, V, K] (NULL = zeros / not stored; ht may be h0), or a pool
 * [pool_slots, H, V, K] with device int32 state_slots [n_seqs] (slot <= 0 or
 * >= pool_slots: zero start, no write; active slots distinct), updated in place.
 * Results in float32; o in bfloat16 is round-to-nearest-even of the float32
 * result. An empty sequence passes its initial state to its final state.
 *
 * Returns GDN_EUNSUPPORTED for K outside {64, 128}, V not a multiple of 16 in
 * [16, 256] or an unknown dtype; GDN_EINVAL for n_seqs < 0, total_tokens < 0, H
 * outside [1, 65535], a non-finite scale, inconsistent offsets or lengths, a
 * NULL input or output when total_tokens > 0, a pool with h0 or ht, a misaligned
 * pointer, or sizes whose grid would not fit; GDN_EWORKSPACE for a missing,
 * small or misaligned workspace; GDN_OK without launching for n_seqs == 0 and
 * total_tokens == 0; GDN_EHIP if a launch fails.
 */
gdn_status gdn_chunk_fwd_kda(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, void* o, int n_seqs, int64_t total_tokens, int H,
                             int K, int V, float scale, gdn_dtype in_dtype, gdn_dtype out_dtype,
                             const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                             const float* h0, float* ht, float* state_pool, int64_t pool_slots,
                             const int32_t* state_slots, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Diagnostic variant of gdn_chunk_fwd_kda for measurement: same arguments and
 * results; in addition it records three caller-created HIP events (hipEvent_t,
 * passed as void*) on `stream`: events[0] before the first kernel, events[1]
 * after the prep kernel, events[2] after the scan. GDN_EINVAL if events or one
 * of them is NULL.
 */
gdn_status gdn_chunk_fwd_kda_profiled(const void* q, const void* k, const void* v, const float* g,
                                      const float* beta, void* o, int n_seqs, int64_t total_tokens,
                                      int H, int K, int V, float scale, gdn_dtype in_dtype,
                                      gdn_dtype out_dtype, const int32_t* cu_seqlens,
                                      const int32_t* cu_seqlens_host, const float* h0, float* ht,
                                      float* state_pool, int64_t pool_slots,
                                      const int32_t* state_slots, void* workspace,
                                      size_t workspace_bytes, void* stream, void* const* events);

/* Static, human-readable name of a status code. Never NULL. */
const char* gdn_status_string(gdn_status s);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */

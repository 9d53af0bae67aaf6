// C ABI of the gated delta rule library: host-side argument validation,
// workspace carving and the launch sequence. Declarations and contracts are in
// include/gdn.h.
#include <limits.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_internal.h"
#include <cmath>
#include <mutex>

namespace {

constexpr int64_t kChunkTokens = 64;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_dim(int d) { return d == 64 || d == 128; }

bool valid_dtype(gdn_dtype t) { return t == GDN_BF16 || t == GDN_F32; }

size_t dtype_bytes(gdn_dtype t) { return t == GDN_F32 ? 4 : 2; }

// Upper bound on the number of chunks of any split of total_tokens into n_seqs
// sequences: sum ceil(len / 64) <= total / 64 + n_seqs.
int64_t max_chunks(int n_seqs, int64_t total_tokens) { return total_tokens / kChunkTokens + n_seqs; }

gdn_status hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_EHIP; }

// Compute units of the current device, asked once per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static int cus[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev >= kMaxDevices) dev = kMaxDevices - 1;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK:
      return "GDN_OK";
    case GDN_EINVAL:
      return "GDN_EINVAL: invalid argument";
    case GDN_EUNSUPPORTED:
      return "GDN_EUNSUPPORTED: unsupported head size or dtype";
    case GDN_EWORKSPACE:
      return "GDN_EWORKSPACE: workspace missing or too small";
    case GDN_EHIP:
      return "GDN_EHIP: HIP runtime error at launch";
  }
  return "GDN_UNKNOWN_STATUS";
}

size_t gdn_chunk_fwd_workspace_bytes(int n_seqs, int64_t total_tokens, int H, int K, int V,
                                     gdn_dtype in_dtype) {
  if (n_seqs < 0 || total_tokens < 0 || H <= 0 || !supported_dim(K) || !supported_dim(V) ||
      !valid_dtype(in_dtype))
    return 0;
  return gdn::workspace_layout(max_chunks(n_seqs, total_tokens), n_seqs, H, K, V, in_dtype == GDN_F32)
      .total;
}

gdn_status gdn_chunk_fwd_plan(int n_seqs, int64_t total_tokens, int64_t max_len, int H, int K, int V,
                              gdn_dtype in_dtype, int32_t* plan, int64_t* offsets) {
  // (the size limits of gdn_chunk_fwd, so that a plan exists only for a call that can be made)
  if (!plan || !offsets || n_seqs < 0 || total_tokens < 0 || max_len < 0 || max_len > total_tokens || H <= 0 ||
      H > 65535 || (n_seqs == 0 && total_tokens > 0) || total_tokens > INT_MAX - 2 * kChunkTokens ||
      static_cast<int64_t>(n_seqs) * H > INT_MAX / 8 ||
      (max_chunks(n_seqs, total_tokens) + 7) / 8 * 8 * H > INT_MAX)
    return GDN_EINVAL;
  if (!supported_dim(K) || !supported_dim(V) || !valid_dtype(in_dtype)) return GDN_EUNSUPPORTED;
  const int64_t max_nc = (max_len + kChunkTokens - 1) / kChunkTokens;
  if (max_nc > INT32_MAX) return GDN_EINVAL;
  const gdn::SegPlan sp = gdn::segment_plan(static_cast<int64_t>(n_seqs) * H, K, V, in_dtype == GDN_F32,
                                            static_cast<int>(max_nc));
  const gdn::WsLayout l =
      gdn::workspace_layout(max_chunks(n_seqs, total_tokens), n_seqs, H, K, V, in_dtype == GDN_F32);
  plan[0] = sp.n_seg;
  plan[1] = sp.L0;
  plan[2] = sp.L1;
  offsets[0] = static_cast<int64_t>(l.af);
  offsets[1] = static_cast<int64_t>(l.pf);
  offsets[2] = static_cast<int64_t>(l.gx);
  offsets[3] = static_cast<int64_t>(l.seg_sum);
  offsets[4] = static_cast<int64_t>(l.seg_state);
  return GDN_OK;
}

}  // extern "C"

namespace {

gdn_status chunk_fwd_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          void* o, int n_seqs, int64_t total_tokens, int H, int K, int V, float scale,
                          gdn_dtype in_dtype, gdn_dtype out_dtype, const int32_t* cu_seqlens,
                          const int32_t* cu_seqlens_host, const float* h0, float* ht, float* state_pool,
                          int64_t pool_slots, const int32_t* state_slots, void* workspace,
                          size_t workspace_bytes, void* stream, void* const* events) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype) || !supported_dim(K) || !supported_dim(V))
    return GDN_EUNSUPPORTED;
  if (n_seqs < 0 || total_tokens < 0 || H <= 0 || H > 65535) return GDN_EINVAL;
  if (total_tokens > INT_MAX - 2 * kChunkTokens) return GDN_EINVAL;
  if (n_seqs == 0) return total_tokens == 0 ? GDN_OK : GDN_EINVAL;
  if ((cu_seqlens == nullptr) != (cu_seqlens_host == nullptr)) return GDN_EINVAL;
  if (static_cast<int64_t>(n_seqs) * H > INT_MAX / 8) return GDN_EINVAL;
  if ((max_chunks(n_seqs, total_tokens) + 7) / 8 * 8 * H > INT_MAX) return GDN_EINVAL;  // prep's grid

  // Chunk count and sequence lengths.
  int64_t n_chunks = 0, max_nc = 0;
  int T_eq = 0;
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] != 0 || cu_seqlens_host[n_seqs] != total_tokens) return GDN_EINVAL;
    for (int s = 0; s < n_seqs; ++s) {
      const int64_t len = static_cast<int64_t>(cu_seqlens_host[s + 1]) - cu_seqlens_host[s];
      if (len < 0) return GDN_EINVAL;
      const int64_t nc = (len + kChunkTokens - 1) / kChunkTokens;
      n_chunks += nc;
      max_nc = nc > max_nc ? nc : max_nc;
    }
  } else {
    if (total_tokens % n_seqs != 0) return GDN_EINVAL;
    T_eq = static_cast<int>(total_tokens / n_seqs);
    max_nc = (T_eq + kChunkTokens - 1) / kChunkTokens;
    n_chunks = static_cast<int64_t>(n_seqs) * max_nc;
  }
  if (n_chunks > INT_MAX) return GDN_EINVAL;

  // Tensors.
  if (total_tokens > 0) {
    if (!q || !k || !v || !g || !beta || !o) return GDN_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return GDN_EINVAL;
    if (!aligned(g, 4) || !aligned(beta, 4)) return GDN_EINVAL;
  }

  // State source and destination.
  if (state_pool) {
    if (h0 || ht || !state_slots || pool_slots <= 0 || !aligned(state_pool, 16)) return GDN_EINVAL;
  } else {
    if (state_slots) return GDN_EINVAL;
    if ((h0 && !aligned(h0, 16)) || (ht && !aligned(ht, 16))) return GDN_EINVAL;
  }

  // Workspace.
  const gdn::WsLayout layout =
      gdn::workspace_layout(max_chunks(n_seqs, total_tokens), n_seqs, H, K, V, in_dtype == GDN_F32);
  if (!workspace || workspace_bytes < layout.total || !aligned(workspace, 256)) return GDN_EWORKSPACE;

  gdn::ChunkArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.n_seqs = n_seqs;
  a.total_tokens = total_tokens;
  a.H = H;
  a.K = K;
  a.V = V;
  a.scale = scale;
  a.in_f32 = in_dtype == GDN_F32;
  a.out_f32 = out_dtype == GDN_F32;
  a.cu_seqlens = cu_seqlens;
  a.n_chunks = n_chunks;
  a.max_nc = static_cast<int>(max_nc);
  a.T_eq = T_eq;
  a.h0 = h0;
  a.ht = ht;
  a.pool = state_pool;
  a.pool_slots = pool_slots;
  a.slots = state_slots;
  a.ws = gdn::carve_workspace(layout, workspace);
  a.n_cus = device_cus();
  a.stream = static_cast<hipStream_t>(stream);
  for (int i = 0; i < 3; ++i) a.events[i] = events ? static_cast<hipEvent_t>(events[i]) : nullptr;
  return hip_status(gdn::launch_chunk_fwd(a));
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         void* o, int n_seqs, int64_t total_tokens, int H, int K, int V, float scale,
                         gdn_dtype in_dtype, gdn_dtype out_dtype, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_host, const float* h0, float* ht, float* state_pool,
                         int64_t pool_slots, const int32_t* state_slots, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl(q, k, v, g, beta, o, n_seqs, total_tokens, H, K, V, scale, in_dtype, out_dtype,
                        cu_seqlens, cu_seqlens_host, h0, ht, state_pool, pool_slots, state_slots, workspace,
                        workspace_bytes, stream, nullptr);
}

gdn_status gdn_chunk_fwd_profiled(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, void* o, int n_seqs, int64_t total_tokens, int H, int K,
                                  int V, float scale, gdn_dtype in_dtype, gdn_dtype out_dtype,
                                  const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, const float* h0,
                                  float* ht, float* state_pool, int64_t pool_slots, const int32_t* state_slots,
                                  void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  if (!events || !events[0] || !events[1] || !events[2]) return GDN_EINVAL;
  return chunk_fwd_impl(q, k, v, g, beta, o, n_seqs, total_tokens, H, K, V, scale, in_dtype, out_dtype,
                        cu_seqlens, cu_seqlens_host, h0, ht, state_pool, pool_slots, state_slots, workspace,
                        workspace_bytes, stream, events);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// gdn_chunk_fwd_noalloc: gdn_chunk_fwd with its workspace in a file-scope
// device array instead of a caller buffer. Each GPU the library runs on holds
// its own copy of the array (GDN_NOALLOC_WORKSPACE_BYTES) until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory:
// the array's device address is asked of the runtime once per device (with
// that device current) and only that address is ever handed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[GDN_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's copy of `scratch` (nullptr on error).
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                 void* o, int n_seqs, int64_t total_tokens, int H, int K, int V, float scale,
                                 gdn_dtype in_dtype, gdn_dtype out_dtype, const int32_t* cu_seqlens,
                                 const int32_t* cu_seqlens_host, const float* h0, float* ht, float* state_pool,
                                 int64_t pool_slots, const int32_t* state_slots, void* stream) {
  // Validation first, without a workspace: an error other than the missing
  // workspace (or a call with nothing to do) returns here, before the device is
  // touched; sizes that need more than the array holds get GDN_EWORKSPACE.
  const gdn_status st = chunk_fwd_impl(q, k, v, g, beta, o, n_seqs, total_tokens, H, K, V, scale, in_dtype,
                                       out_dtype, cu_seqlens, cu_seqlens_host, h0, ht, state_pool, pool_slots,
                                       state_slots, nullptr, 0, stream, nullptr);
  if (st != GDN_EWORKSPACE) return st;
  const size_t need = gdn_chunk_fwd_workspace_bytes(n_seqs, total_tokens, H, K, V, in_dtype);
  if (need == 0 || need > GDN_NOALLOC_WORKSPACE_BYTES) return GDN_EWORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return GDN_EHIP;
  return chunk_fwd_impl(q, k, v, g, beta, o, n_seqs, total_tokens, H, K, V, scale, in_dtype, out_dtype,
                        cu_seqlens, cu_seqlens_host, h0, ht, state_pool, pool_slots, state_slots, ws,
                        GDN_NOALLOC_WORKSPACE_BYTES, stream, nullptr);
}

}  // extern "C"

namespace {

gdn_status recurrent_step_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                               float* state_pool, int64_t pool_slots, const int32_t* slots, void* o, int N, int H,
                               int K, int V, float scale, gdn_dtype in_dtype, gdn_dtype out_dtype, void* stream,
                               bool kda) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype) || !supported_dim(K) || !supported_dim(V))
    return GDN_EUNSUPPORTED;
  if (N < 0 || H <= 0 || H > 65535) return GDN_EINVAL;
  // one workgroup per 16 state rows of each (request, head), in a 1-D grid
  if (static_cast<int64_t>(N) * H * (V / 16) > INT32_MAX) return GDN_EINVAL;
  if (N == 0) return GDN_OK;
  if (!q || !k || !v || !g || !beta || !state_pool || !slots || !o || pool_slots <= 0) return GDN_EINVAL;
  if (!aligned(state_pool, 16) || !aligned(g, kda ? 16 : 4) || !aligned(beta, 4) || !aligned(slots, 4))
    return GDN_EINVAL;
  const size_t in_b = dtype_bytes(in_dtype), out_b = dtype_bytes(out_dtype);
  if (!aligned(q, in_b) || !aligned(k, in_b) || !aligned(v, in_b) || !aligned(o, out_b)) return GDN_EINVAL;

  gdn::DecodeArgs a{};
  a.kda = kda;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.pool = state_pool;
  a.pool_slots = pool_slots;
  a.slots = slots;
  a.o = o;
  a.N = N;
  a.H = H;
  a.K = K;
  a.V = V;
  a.scale = scale;
  a.in_f32 = in_dtype == GDN_F32;
  a.out_f32 = out_dtype == GDN_F32;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(gdn::launch_decode(a));
}

}  // namespace

extern "C" {

gdn_status gdn_recurrent_step(const void* q, const void* k, const void* v, const float* g, const float* beta,
                              float* state_pool, int64_t pool_slots, const int32_t* slots, void* o, int N, int H,
                              int K, int V, float scale, gdn_dtype in_dtype, gdn_dtype out_dtype, void* stream) {
  return recurrent_step_impl(q, k, v, g, beta, state_pool, pool_slots, slots, o, N, H, K, V, scale, in_dtype,
                             out_dtype, stream, false);
}

gdn_status gdn_recurrent_step_kda(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                  float* state_pool, int64_t pool_slots, const int32_t* slots, void* o, int N, int H,
                                  int K, int V, float scale, gdn_dtype in_dtype, gdn_dtype out_dtype, void* stream) {
  return recurrent_step_impl(q, k, v, g, beta, state_pool, pool_slots, slots, o, N, H, K, V, scale, in_dtype,
                             out_dtype, stream, true);
}


gdn_status gdn_recurrent_verify(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                float* state_pool, int64_t pool_slots, const int32_t* slots, int slot_cols,
                                const int32_t* accepted, void* o, int N, int T, int H, int K, int V, float scale,
                                gdn_dtype in_dtype, gdn_dtype out_dtype, void* stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype) || !supported_dim(K) || !supported_dim(V))
    return GDN_EUNSUPPORTED;
  if (N < 0 || H <= 0 || H > 65535 || T < 1 || T > 8 || slot_cols < T) return GDN_EINVAL;
  if (static_cast<int64_t>(N) * H * (V / 16) > INT32_MAX) return GDN_EINVAL;
  if (static_cast<int64_t>(N) * T * H > INT32_MAX / 128) return GDN_EINVAL;
  if (N == 0) return GDN_OK;
  if (!q || !k || !v || !g || !beta || !state_pool || !slots || !accepted || !o || pool_slots <= 0)
    return GDN_EINVAL;
  if (!aligned(state_pool, 16) || !aligned(g, 4) || !aligned(beta, 4) || !aligned(slots, 4) || !aligned(accepted, 4))
    return GDN_EINVAL;
  const size_t in_b = dtype_bytes(in_dtype), out_b = dtype_bytes(out_dtype);
  if (!aligned(q, in_b) || !aligned(k, in_b) || !aligned(v, in_b) || !aligned(o, out_b)) return GDN_EINVAL;

  gdn::VerifyArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.pool = state_pool;
  a.pool_slots = pool_slots;
  a.slots = slots;
  a.cols = slot_cols;
  a.accepted = accepted;
  a.o = o;
  a.N = N;
  a.T = T;
  a.H = H;
  a.K = K;
  a.V = V;
  a.scale = scale;
  a.in_f32 = in_dtype == GDN_F32;
  a.out_f32 = out_dtype == GDN_F32;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(gdn::launch_verify(a));
}


gdn_status gdn_kda_gate(const void* f_a, const void* f_b, const float* a_log, const float* dt_bias,
                        float lower_bound, int mode, float* g, void* raw_g, int N, int H, int K, void* stream) {
  if (K != 64 && K != 128) return GDN_EUNSUPPORTED;
  if (mode < 0 || mode > 2 || N < 0 || H <= 0 || H > 65535 || !std::isfinite(lower_bound)) return GDN_EINVAL;
  if (static_cast<int64_t>(N) * H * K > INT64_MAX / 4) return GDN_EINVAL;
  // one workgroup per (8 tokens, head), heads padded to multiples of 8: a 1-D grid
  if ((static_cast<int64_t>(N) + 7) / 8 * ((H + 7) / 8) * 8 > INT32_MAX) return GDN_EINVAL;
  if (N == 0) return GDN_OK;
  if (!f_a || !f_b || !a_log || !dt_bias || !g) return GDN_EINVAL;
  if (!aligned(f_a, 16) || !aligned(f_b, 16) || !aligned(a_log, 4) || !aligned(dt_bias, 4) || !aligned(g, 4) ||
      (raw_g && !aligned(raw_g, 2)))
    return GDN_EINVAL;
  gdn::GateArgs a{};
  a.f_a = f_a;
  a.f_b = f_b;
  a.a_log = a_log;
  a.dt_bias = dt_bias;
  a.lower_bound = lower_bound;
  a.mode = mode;
  a.g = g;
  a.raw_out = raw_g;
  a.N = N;
  a.H = H;
  a.K = K;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(gdn::launch_kda_gate(a));
}

gdn_status gdn_fp8_quant(const float* x, void* codes, float* scales, int64_t rows, int64_t cols, int group,
                         void* stream) {
  if (group != 64 && group != 128) return GDN_EUNSUPPORTED;
  if (rows < 0 || cols < 0 || cols % group != 0) return GDN_EINVAL;
  if (cols > 0 && rows > INT64_MAX / cols) return GDN_EINVAL;
  const int64_t n_groups = rows * (cols / group);
  // one workgroup per 32 (group 128) or 64 (group 64) groups in a 1-D grid
  if (n_groups / (group == 128 ? 32 : 64) >= INT32_MAX) return GDN_EINVAL;
  if (n_groups == 0) return GDN_OK;
  if (!x || !codes || !scales) return GDN_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(scales, 4)) return GDN_EINVAL;
  gdn::Fp8Args a{};
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  a.n_groups = n_groups;
  a.group = group;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(gdn::launch_fp8_quant(a));
}


gdn_status gdn_decode_prologue(const void* x, const float* conv_w, const float* conv_bias, void* conv_state,
                               int64_t pool_slots, const int32_t* slots, const float* beta_raw, float* q, float* k,
                               float* v, float* beta, int N, int H, int D, void* stream) {
  if (D != 64 && D != 128) return GDN_EUNSUPPORTED;
  if (N < 0 || H <= 0 || H > 65535 || static_cast<int64_t>(N) * H > INT32_MAX) return GDN_EINVAL;
  if (N == 0) return GDN_OK;
  if (!x || !conv_w || !conv_state || !slots || !beta_raw || !q || !k || !v || !beta || pool_slots <= 0)
    return GDN_EINVAL;
  if (!aligned(x, 4) || !aligned(conv_state, 4) || !aligned(conv_w, 8) || !aligned(slots, 4) ||
      !aligned(beta_raw, 4) || !aligned(q, 8) || !aligned(k, 8) || !aligned(v, 8) || !aligned(beta, 4) ||
      (conv_bias && !aligned(conv_bias, 8)))
    return GDN_EINVAL;
  gdn::PrologueArgs a{};
  a.x = x;
  a.conv_w = conv_w;
  a.conv_bias = conv_bias;
  a.conv_state = conv_state;
  a.pool_slots = pool_slots;
  a.slots = slots;
  a.beta_raw = beta_raw;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.N = N;
  a.H = H;
  a.D = D;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(gdn::launch_decode_prologue(a));
}

gdn_status gdn_decode_prologue_verify(const void* x, const float* conv_w, const float* conv_bias, void* conv_state,
                                      int64_t pool_slots, const int32_t* slots, int slot_cols,
                                      const int32_t* accepted, const float* beta_raw, float* q, float* k, float* v,
                                      float* beta, int N, int T, int H, int D, void* stream) {
  if (D != 64 && D != 128) return GDN_EUNSUPPORTED;
  if (N < 0 || T < 1 || T > 8 || slot_cols < T || H <= 0 || H > 65535) return GDN_EINVAL;
  if (static_cast<int64_t>(N) * H * (D / 2) > INT32_MAX || static_cast<int64_t>(N) * T * H > INT32_MAX)
    return GDN_EINVAL;
  if (N == 0) return GDN_OK;
  if (!x || !conv_w || !conv_state || !slots || !accepted || !beta_raw || !q || !k || !v || !beta ||
      pool_slots <= 0)
    return GDN_EINVAL;
  if (!aligned(x, 4) || !aligned(conv_state, 2) || !aligned(conv_w, 8) || !aligned(slots, 4) ||
      !aligned(accepted, 4) || !aligned(beta_raw, 4) || !aligned(q, 8) || !aligned(k, 8) || !aligned(v, 8) ||
      !aligned(beta, 4) || (conv_bias && !aligned(conv_bias, 8)))
    return GDN_EINVAL;
  gdn::PrologueArgs a{};
  a.x = x;
  a.conv_w = conv_w;
  a.conv_bias = conv_bias;
  a.conv_state = conv_state;
  a.pool_slots = pool_slots;
  a.slots = slots;
  a.cols = slot_cols;
  a.accepted = accepted;
  a.beta_raw = beta_raw;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.N = N;
  a.T = T;
  a.H = H;
  a.D = D;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(gdn::launch_decode_prologue_verify(a));
}

gdn_status gdn_decode_layer(const void* x, const float* conv_w, const float* conv_bias, void* conv_state,
                            int64_t conv_slots, const int32_t* slots, const float* beta_raw, const float* g,
                            int g_per_channel, float* state_pool, int64_t pool_slots, const void* gate,
                            const float* norm_w, float eps, void* out, gdn_dtype out_dtype, int N, int H, int D,
                            float scale, void* stream) {
  if (D != 64 && D != 128) return GDN_EUNSUPPORTED;
  if (!valid_dtype(out_dtype)) return GDN_EUNSUPPORTED;
  if (N < 0 || H <= 0 || H > 65535 || static_cast<int64_t>(N) * H > INT32_MAX) return GDN_EINVAL;
  if (norm_w && !(eps >= 0.f)) return GDN_EINVAL;
  if (N == 0) return GDN_OK;
  if (!x || !conv_w || !conv_state || !slots || !beta_raw || !g || !state_pool || !out || conv_slots <= 0 ||
      pool_slots <= 0 || (norm_w && !gate))
    return GDN_EINVAL;
  if (!aligned(x, 2) || !aligned(conv_state, 2) || !aligned(conv_w, 4) || !aligned(slots, 4) ||
      !aligned(beta_raw, 4) || !aligned(g, g_per_channel ? 16 : 4) || !aligned(state_pool, 16) ||
      !aligned(out, dtype_bytes(out_dtype)) || (conv_bias && !aligned(conv_bias, 4)) ||
      (norm_w && (!aligned(norm_w, 4) || !aligned(gate, 2))))
    return GDN_EINVAL;
  gdn::LayerArgs a{};
  a.x = x;
  a.conv_w = conv_w;
  a.conv_bias = conv_bias;
  a.conv_state = conv_state;
  a.conv_slots = conv_slots;
  a.slots = slots;
  a.beta_raw = beta_raw;
  a.g = g;
  a.kda = g_per_channel != 0;
  a.pool = state_pool;
  a.pool_slots = pool_slots;
  a.gate = gate;
  a.norm_w = norm_w;
  a.eps = eps;
  a.out = out;
  a.out_f32 = out_dtype == GDN_F32;
  a.N = N;
  a.H = H;
  a.D = D;
  a.scale = scale;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(gdn::launch_decode_layer(a));
}

gdn_status gdn_gated_rmsnorm(const float* o, const void* gate, const float* norm_w, float eps, void* out, int N, int H,
                             int D, gdn_dtype out_dtype, void* stream) {
  if (D != 64 && D != 128) return GDN_EUNSUPPORTED;
  if (!valid_dtype(out_dtype)) return GDN_EUNSUPPORTED;
  if (N < 0 || H <= 0 || H > 65535 || static_cast<int64_t>(N) * H > INT32_MAX || !(eps >= 0.f)) return GDN_EINVAL;
  if (N == 0) return GDN_OK;
  if (!o || !gate || !norm_w || !out) return GDN_EINVAL;
  if (!aligned(o, 8) || !aligned(gate, 4) || !aligned(norm_w, 8) || !aligned(out, 2 * dtype_bytes(out_dtype)))
    return GDN_EINVAL;
  gdn::RmsNormArgs a{};
  a.o = o;
  a.gate = gate;
  a.norm_w = norm_w;
  a.eps = eps;
  a.out = out;
  a.out_f32 = out_dtype == GDN_F32;
  a.N = N;
  a.H = H;
  a.D = D;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(gdn::launch_gated_rmsnorm(a));
}


size_t gdn_chunk_fwd_kda_workspace_bytes(int n_seqs, int64_t total_tokens, int H, int K) {
  if (n_seqs < 0 || total_tokens < 0 || H <= 0 || H > 65535 || (K != 64 && K != 128)) return 0;
  return gdn::kda_workspace_bytes(max_chunks(n_seqs, total_tokens), n_seqs, H, K);
}

static gdn_status chunk_fwd_kda_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                     void* o, int n_seqs, int64_t total_tokens, int H, int K, int V, float scale,
                                     gdn_dtype in_dtype, gdn_dtype out_dtype, const int32_t* cu_seqlens,
                                     const int32_t* cu_seqlens_host, const float* h0, float* ht, float* state_pool,
                                     int64_t pool_slots, const int32_t* state_slots, void* workspace,
                                     size_t workspace_bytes, void* stream, void* const* events) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype) || (K != 64 && K != 128) || V % 16 != 0 || V < 16 ||
      V > 256)
    return GDN_EUNSUPPORTED;
  if (n_seqs < 0 || total_tokens < 0 || H <= 0 || H > 65535 || !std::isfinite(scale)) return GDN_EINVAL;
  if (total_tokens > INT_MAX - 2 * kChunkTokens) return GDN_EINVAL;
  if (n_seqs == 0) return total_tokens == 0 ? GDN_OK : GDN_EINVAL;
  if ((cu_seqlens == nullptr) != (cu_seqlens_host == nullptr)) return GDN_EINVAL;
  if ((static_cast<int64_t>(n_seqs) * H + 7) / 8 * 8 * (V / 16) > INT32_MAX) return GDN_EINVAL;
  int64_t n_chunks = 0;
  int T_eq = 0;
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] != 0 || cu_seqlens_host[n_seqs] != total_tokens) return GDN_EINVAL;
    for (int s = 0; s < n_seqs; ++s) {
      const int64_t len = static_cast<int64_t>(cu_seqlens_host[s + 1]) - cu_seqlens_host[s];
      if (len < 0) return GDN_EINVAL;
      n_chunks += (len + kChunkTokens - 1) / kChunkTokens;
    }
  } else {
    if (total_tokens % n_seqs != 0) return GDN_EINVAL;
    T_eq = static_cast<int>(total_tokens / n_seqs);
    n_chunks = static_cast<int64_t>(n_seqs) * ((T_eq + kChunkTokens - 1) / kChunkTokens);
  }
  if (n_chunks > INT_MAX) return GDN_EINVAL;
  if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_EINVAL;
  const size_t in_b = dtype_bytes(in_dtype), out_b = dtype_bytes(out_dtype);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, in_b) || !aligned(g, 16) || !aligned(beta, 4) ||
      !aligned(o, out_b))
    return GDN_EINVAL;
  if (state_pool) {
    if (h0 || ht || !state_slots || pool_slots <= 0 || !aligned(state_pool, 4) || !aligned(state_slots, 4))
      return GDN_EINVAL;
  } else {
    if (state_slots || !aligned(h0, 4) || !aligned(ht, 4)) return GDN_EINVAL;
  }
  const size_t need = gdn_chunk_fwd_kda_workspace_bytes(n_seqs, total_tokens, H, K);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return GDN_EWORKSPACE;
  gdn::KdaChunkArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.n_seqs = n_seqs;
  a.total_tokens = total_tokens;
  a.H = H;
  a.K = K;
  a.V = V;
  a.scale = scale;
  a.in_f32 = in_dtype == GDN_F32;
  a.out_f32 = out_dtype == GDN_F32;
  a.cu_seqlens = cu_seqlens;
  a.n_chunks = n_chunks;
  a.T_eq = T_eq;
  a.h0 = h0;
  a.ht = ht;
  a.pool = state_pool;
  a.pool_slots = pool_slots;
  a.slots = state_slots;
  a.ws = workspace;
  a.stream = static_cast<hipStream_t>(stream);
  for (int i = 0; i < 3; ++i) a.events[i] = events ? static_cast<hipEvent_t>(events[i]) : nullptr;
  return hip_status(gdn::launch_chunk_fwd_kda(a));
}

gdn_status gdn_chunk_fwd_kda(const void* q, const void* k, const void* v, const float* g, const float* beta, void* o,
                             int n_seqs, int64_t total_tokens, int H, int K, int V, float scale, gdn_dtype in_dtype,
                             gdn_dtype out_dtype, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                             const float* h0, float* ht, float* state_pool, int64_t pool_slots,
                             const int32_t* state_slots, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_fwd_kda_impl(q, k, v, g, beta, o, n_seqs, total_tokens, H, K, V, scale, in_dtype, out_dtype,
                            cu_seqlens, cu_seqlens_host, h0, ht, state_pool, pool_slots, state_slots, workspace,
                            workspace_bytes, stream, nullptr);
}

gdn_status gdn_chunk_fwd_kda_profiled(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                      void* o, int n_seqs, int64_t total_tokens, int H, int K, int V, float scale,
                                      gdn_dtype in_dtype, gdn_dtype out_dtype, const int32_t* cu_seqlens,
                                      const int32_t* cu_seqlens_host, const float* h0, float* ht,
                                      float* state_pool, int64_t pool_slots, const int32_t* state_slots,
                                      void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  if (!events || !events[0] || !events[1] || !events[2]) return GDN_EINVAL;
  return chunk_fwd_kda_impl(q, k, v, g, beta, o, n_seqs, total_tokens, H, K, V, scale, in_dtype, out_dtype,
                            cu_seqlens, cu_seqlens_host, h0, ht, state_pool, pool_slots, state_slots, workspace,
                            workspace_bytes, stream, events);
}

}  // extern "C"
